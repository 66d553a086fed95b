"""Seeded synthetic layer inputs (weights, activations, calibration tokens).

This module only draws random numbers and rounds them to fp16.  It holds none
of the quantisation arithmetic, so both the CPU oracle's tests and the HIP
path can take their inputs from it.

The pages evaluate on LLaMA3 and Qwen3 checkpoints and an unnamed perplexity
set (MosaicQuant technical summary, gist.science/pt/paper/2606.15652,
"Resultados Experimentais").  Neither weights nor data are available here, so
these generators stand in for them with the layer shapes of those models and
value distributions that carry the property the method targets: a few
large-magnitude input channels in the weights and in the activations
(MosaicQuant summary, "Declaração do Problema": rare large-magnitude outliers
beside dense inliers).

Recipe (all draws in float64, then cast to fp16 with round-to-nearest-even):
  * every stream is ``numpy.random.default_rng([seed, role, *dims])`` so a
    tensor depends only on the seed, its role and its own shape;
  * weights ``normal``: N(0, 0.02^2); ``student_t``: 0.02 * t(nu=3)/sqrt(3)
    (unit-variance heavy tail scaled to std 0.02);
  * weight outlier input channels: ``round(frac*K)`` distinct columns drawn
    without replacement, multiplied by ``w_outlier_mult``;
  * activations: N(0, 1) with a fixed set of outlier input channels shared by
    evaluation and calibration tokens, each scaled by a per-channel factor
    (a constant, or uniform in [lo, hi]);
  * calibration tokens use the same channel set as the evaluation tokens but
    an independent stream.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

import numpy as np

ROLE_W = 1
ROLE_X = 2
ROLE_XC = 3
ROLE_CHAN_W = 4
ROLE_CHAN_X = 5
ROLE_CHAN_SCALE = 6


@dataclass(frozen=True)
class LayerSpec:
    """Shape and value distribution of one synthetic linear layer."""
    name: str
    K: int                       # input channels
    N: int                       # output channels
    w_kind: str = "normal"       # "normal" | "student_t"
    w_std: float = 0.02
    w_outlier_frac: float = 0.0  # fraction of input channels scaled up in W
    w_outlier_mult: float = 20.0
    x_outlier_count: int = -1    # -1: round(x_outlier_frac * K)
    x_outlier_frac: float = 0.01
    x_outlier_scale: Tuple[float, float] = (10.0, 50.0)  # (c, c) = constant
    T: int = 512                 # calibration tokens
    block: int = 64              # residual block edge
    rho: float = 0.10            # residual budget (fraction of blocks)

    @property
    def n_blocks(self) -> int:
        return (self.N // self.block) * (self.K // self.block)

    @property
    def n_select(self) -> int:
        # floor(rho * B): the budget is never exceeded
        return int(np.floor(self.rho * self.n_blocks + 1e-9))

    def with_block(self, block: int, rho: float | None = None) -> "LayerSpec":
        return LayerSpec(**{**self.__dict__, "block": block,
                            "rho": self.rho if rho is None else rho})


def _rng(seed: int, role: int, *dims: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(role)] + [int(d) for d in dims])


def _to_f16(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def weight_outlier_channels(spec: LayerSpec, seed: int = 0) -> np.ndarray:
    n = int(round(spec.w_outlier_frac * spec.K))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    r = _rng(seed, ROLE_CHAN_W, spec.K, spec.N)
    return np.sort(r.choice(spec.K, size=n, replace=False))


def act_outlier_channels(spec: LayerSpec, seed: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """(channel indices, per-channel multipliers), shared by X and Xc."""
    n = spec.x_outlier_count if spec.x_outlier_count >= 0 else int(round(spec.x_outlier_frac * spec.K))
    if n == 0:
        return np.zeros(0, dtype=np.int64), np.zeros(0)
    idx = np.sort(_rng(seed, ROLE_CHAN_X, spec.K).choice(spec.K, size=n, replace=False))
    lo, hi = spec.x_outlier_scale
    if lo == hi:
        mult = np.full(n, float(lo))
    else:
        mult = _rng(seed, ROLE_CHAN_SCALE, spec.K).uniform(lo, hi, size=n)
    return idx, mult


def make_weight(spec: LayerSpec, seed: int = 0) -> np.ndarray:
    """fp16 [N, K] weight (rows = output channels)."""
    r = _rng(seed, ROLE_W, spec.K, spec.N)
    if spec.w_kind == "normal":
        w = r.standard_normal((spec.N, spec.K)) * spec.w_std
    elif spec.w_kind == "student_t":
        w = r.standard_t(3.0, size=(spec.N, spec.K)) * (spec.w_std / np.sqrt(3.0))
    else:
        raise ValueError(f"unknown weight kind {spec.w_kind!r}")
    ch = weight_outlier_channels(spec, seed)
    if ch.size:
        w[:, ch] *= spec.w_outlier_mult
    return _to_f16(w)


def _acts(spec: LayerSpec, rows: int, seed: int, role: int) -> np.ndarray:
    x = _rng(seed, role, rows, spec.K).standard_normal((rows, spec.K))
    idx, mult = act_outlier_channels(spec, seed)
    if idx.size:
        x[:, idx] *= mult[None, :]
    return _to_f16(x)


def make_acts(spec: LayerSpec, M: int, seed: int = 0) -> np.ndarray:
    """fp16 [M, K] evaluation activations."""
    return _acts(spec, M, seed, ROLE_X)


def make_calib(spec: LayerSpec, seed: int = 0) -> np.ndarray:
    """fp16 [T, K] calibration activations (independent of the evaluation draw)."""
    return _acts(spec, spec.T, seed, ROLE_XC)


# --------------------------------------------------------------------------
# Named layer families (shapes of the models the pages evaluate on)
# --------------------------------------------------------------------------

TINY = LayerSpec("tiny-512x512", K=512, N=512, x_outlier_count=4,
                 x_outlier_scale=(20.0, 20.0), T=64, block=64, rho=0.10)
TINY_M = 16


def llama3_8b(K: int, N: int) -> LayerSpec:
    return LayerSpec(f"llama3-8b-{K}x{N}", K=K, N=N, w_outlier_frac=0.005,
                     w_outlier_mult=20.0, T=512, block=64, rho=0.10)


LLAMA3_8B_SHAPES = [(4096, 4096), (4096, 14336), (14336, 4096)]
LLAMA3_8B_DECODE_M = [1, 4, 16]
LLAMA3_8B_PREFILL_M = 2048


def qwen3_32b(K: int, N: int) -> LayerSpec:
    return LayerSpec(f"qwen3-32b-{K}x{N}", K=K, N=N, w_kind="student_t",
                     T=512, block=64, rho=0.10)


QWEN3_32B_SHAPES = [(5120, 25600), (25600, 5120)]
QWEN3_32B_M = [1, 16, 256, 4096]


def llama3_70b(block: int = 64, rho: float = 0.10) -> LayerSpec:
    return LayerSpec(f"llama3-70b-8192x28672-b{block}-r{int(round(rho*100))}",
                     K=8192, N=28672, w_outlier_frac=0.005, w_outlier_mult=20.0,
                     T=512, block=block, rho=rho)


LLAMA3_70B_M = 256
LLAMA3_70B_BLOCKS = [32, 64, 128]
LLAMA3_70B_RHOS = [0.0, 0.05, 0.10, 0.20]
