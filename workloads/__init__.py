"""Seeded synthetic inputs for the SVDQuant W4A4 linear (FLUX-shaped layers).

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It draws random numbers and rounds them to bf16 storage; it holds
none of the quantization method's arithmetic (no smoothing, SVD, quantizer or
product).  The calibration statistic ``act_absmax`` (per input channel, the
largest |x| over the calibration rows) is part of the input recipe: the pages
calibrate on a dataset that is not available, so the test activations
themselves serve as calibration data.

Shapes follow FLUX.1 at 1024x1024 (4096 image tokens, hidden size 3072, MLP
width 12288); the token count is a multiple of 256 because the model card's
"Model Description" requires the pixel count to be a multiple of 65,536.  The
trained FLUX weights are not available; weights are N(0, 0.02^2) in the
``[out_features][in_features]`` layout of ``torch.nn.Linear``.

Draw order (fixed, per workload, ``numpy.random.default_rng(seed)``):
  1. X ~ N(0, 1) as [M][K] (rows of a second token stream, if any, are
     scaled by its standard deviation), rounded to bf16;
  2. outlier channel indices: ``rng.choice(K, n_out, replace=False)``;
  3. outlier factors (constant, or U[lo, hi]);
  4. those columns multiplied by their factor, re-rounded to bf16;
  5. each weight ~ N(0, 0.02^2) as [N][K], rounded to bf16 (in the order the
     layers are listed);
  6. bias ~ N(0, 0.01^2) as [N], rounded to bf16 (only where a bias exists).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "bf16_bits_from_f32",
    "bf16_bits_to_f64",
    "Layer",
    "Workload",
    "make_workload",
    "custom_workload",
    "WORKLOADS",
]


def bf16_bits_from_f32(a) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Input preparation only: the synthetic draws are stored as bf16 like the
    16-bit activations and weights of a real model.
    """
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f64(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Layer:
    """One linear layer: weight [N][K] (bf16 bits), optional bias [N] (bf16 bits)."""
    name: str
    K: int
    N: int
    weight_bits: np.ndarray
    bias_bits: Optional[np.ndarray] = None

    @property
    def weight(self) -> np.ndarray:
        return bf16_bits_to_f64(self.weight_bits)

    @property
    def bias(self) -> Optional[np.ndarray]:
        return None if self.bias_bits is None else bf16_bits_to_f64(self.bias_bits)


@dataclasses.dataclass
class Workload:
    name: str
    M: int
    x_bits: np.ndarray            # [M][K] bf16 bits
    layers: list                  # list[Layer]
    ranks: tuple                  # ranks exercised on this workload
    group: int = 64
    outlier_channels: Optional[np.ndarray] = None
    outlier_factors: Optional[np.ndarray] = None
    chain_gelu: bool = False      # second layer consumes tanh-GELU of the first's output

    @property
    def x(self) -> np.ndarray:
        return bf16_bits_to_f64(self.x_bits)

    def act_absmax(self) -> np.ndarray:
        """Per-input-channel calibration statistic max_m |X[m, k]| as float32."""
        return np.abs(self.x).max(axis=0).astype(np.float32)


def _draw_activation(rng, M, K, row_std, n_out, factor):
    x = rng.standard_normal((M, K))
    x *= row_std[:, None]
    xb = bf16_bits_from_f32(x.astype(np.float32))
    idx = np.sort(rng.choice(K, n_out, replace=False)) if n_out > 0 else np.zeros(0, np.int64)
    if isinstance(factor, tuple):
        fac = rng.uniform(factor[0], factor[1], n_out)
    else:
        fac = np.full(n_out, float(factor))
    if n_out:
        xv = bf16_bits_to_f64(xb)
        xv[:, idx] *= fac[None, :]
        xb = bf16_bits_from_f32(xv.astype(np.float32))
    return xb, idx, fac


def _draw_weight(rng, N, K, std=0.02):
    return bf16_bits_from_f32((rng.standard_normal((N, K)) * std).astype(np.float32))


def _draw_bias(rng, N, std=0.01):
    return bf16_bits_from_f32((rng.standard_normal(N) * std).astype(np.float32))


def custom_workload(M, K, N, *, seed=0, n_out=4, factor=30.0, bias=False,
                    text_rows=0, text_std=np.sqrt(3.0), ranks=(32,), name=None,
                    second_N=None) -> Workload:
    """Generic recipe used by the FLUX-shaped workloads and by small test shapes.

    ``second_N`` adds a second layer [second_N][N] fed by tanh-GELU of the first
    layer's output (the MLP pair).
    """
    rng = np.random.default_rng(seed)
    row_std = np.ones(M)
    if text_rows:
        # joint stream: the text tokens come first, then the image tokens
        row_std[:text_rows] = text_std
    xb, idx, fac = _draw_activation(rng, M, K, row_std, n_out, factor)
    layers = [Layer("up" if second_N else "linear", K, N, _draw_weight(rng, N, K))]
    if second_N:
        layers.append(Layer("down", N, second_N, _draw_weight(rng, second_N, N)))
    if bias:
        for L in layers:
            L.bias_bits = _draw_bias(rng, L.N)
    return Workload(name or f"custom_{M}x{K}x{N}", M, xb, layers, tuple(ranks),
                    outlier_channels=idx, outlier_factors=fac,
                    chain_gelu=bool(second_N))


# name -> (constructor kwargs, one-line description)
WORKLOADS = {
    "tiny": dict(M=256, K=512, N=512, seed=0, n_out=4, factor=30.0, ranks=(32,)),
    "attn_out": dict(M=4096, K=3072, N=3072, seed=1, n_out=15, factor=(20.0, 50.0), ranks=(32,)),
    "joint_qkv": dict(M=4608, K=3072, N=9216, seed=2, n_out=15, factor=(20.0, 50.0),
                      bias=True, text_rows=512, ranks=(32,)),
    "mlp_pair": dict(M=4096, K=3072, N=12288, seed=3, n_out=15, factor=(20.0, 50.0),
                     second_N=3072, ranks=(32,)),
    "rank_sweep": dict(M=16384, K=3072, N=12288, seed=4, n_out=15, factor=(20.0, 50.0),
                       ranks=(0, 16, 32, 64, 128)),
}

DESCRIPTIONS = {
    "tiny": "single linear 256x512x512, r=32, 4 outlier channels x30",
    "attn_out": "DiT attention-output projection 4096x3072x3072, r=32",
    "joint_qkv": "joint-stream fused QKV 4608x3072x9216 (4096 image + 512 text rows), r=32, bias",
    "mlp_pair": "MLP pair: up 4096x3072x12288 then tanh-GELU, down 4096x12288x3072, r=32",
    "rank_sweep": "batched rank sweep 16384x3072x12288, r in {0,16,32,64,128}",
}


def make_workload(name: str, M: Optional[int] = None) -> Workload:
    """Build a named FLUX-shaped workload.  ``M`` overrides the token count
    (rows are then a prefix-independent fresh draw with the same recipe)."""
    kw = dict(WORKLOADS[name])
    if M is not None:
        if kw.get("text_rows"):
            kw["text_rows"] = max(1, M * kw["text_rows"] // kw["M"])
        kw["M"] = M
    return custom_workload(name=name, **kw)


# --------------------------------------------------------------------------
# Inputs of the fused QKV epilogue (per-head Q/K RMSNorm + rotary embedding)
# --------------------------------------------------------------------------
def rope_tables(text_rows: int, image_side: int, head_dim: int = 128, theta: float = 10000.0,
                axes=(16, 56, 56)):
    """cos / sin tables [M][head_dim/2] (float32) with FLUX's layout of
    positions: text tokens at (0, 0, 0), image tokens at (0, h, w) on an
    image_side x image_side grid; the head dimension is split over three
    position axes of widths ``axes`` and pair j of an axis of width d turns by
    pos * theta^(-2j/d).  These are input data of the operator (the model
    computes them), drawn here with the FLUX-style structure."""
    assert sum(axes) == head_dim
    M = text_rows + image_side * image_side
    pos = np.zeros((M, 3))
    hh, ww = np.meshgrid(np.arange(image_side), np.arange(image_side), indexing="ij")
    pos[text_rows:, 1] = hh.reshape(-1)
    pos[text_rows:, 2] = ww.reshape(-1)
    angles = []
    for a, d in enumerate(axes):
        j = np.arange(d // 2)
        omega = theta ** (-2.0 * j / d)
        angles.append(pos[:, a:a + 1] * omega[None, :])
    ang = np.concatenate(angles, axis=1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def norm_weights(head_dim: int = 128, seed: int = 5):
    """RMSNorm weights for Q and K as bf16 bit patterns and their values:
    1 + N(0, 0.1^2), rounded to bf16."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(2):
        v = (1.0 + 0.1 * rng.standard_normal(head_dim)).astype(np.float32)
        bits = bf16_bits_from_f32(v)
        out.append((bits, bf16_bits_to_f64(bits)))
    return out


# --------------------------------------------------------------------------
# AWQ W4A16 modulation-layer inputs
# --------------------------------------------------------------------------
def _silu(v):
    return v / (1.0 + np.exp(-v))


def awq_workload(M: int, K: int = 3072, N: int = 18432, Mc: int = 32, seed: int = 6, n_out: int = 8):
    """FLUX adaLN modulation projection (conditioning vector -> 6 x hidden).
    Inputs are SiLU of a Gaussian with log-normal per-channel magnitudes
    (exp(N(0, 0.75^2))) and ``n_out`` channels x10, which is what makes the
    activation-aware scaling matter; the calibration rows are ``Mc`` further
    draws of the same distribution.  Weights N(0, 0.02^2) and bias
    N(0, 0.01^2), all rounded to bf16.  Returns a dict of bit patterns and
    values."""
    rng = np.random.default_rng(seed)
    mag = np.exp(0.75 * rng.standard_normal(K))
    mag[rng.choice(K, n_out, replace=False)] *= 10.0
    w = rng.standard_normal((N, K)).astype(np.float32) * 0.02
    b = rng.standard_normal(N).astype(np.float32) * 0.01

    def draw(rows):
        return _silu(rng.standard_normal((rows, K)) * mag[None, :]).astype(np.float32)

    x = draw(M)
    xc = draw(Mc)
    out = {}
    for name, v in (("x", x), ("x_cal", xc), ("weight", w), ("bias", b)):
        bits = bf16_bits_from_f32(v)
        out[name + "_bits"] = bits
        out[name] = bf16_bits_to_f64(bits)
    out.update(M=M, K=K, N=N, Mc=Mc)
    return out
