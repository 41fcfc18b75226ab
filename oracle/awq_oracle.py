"""CPU oracle for the AWQ W4A16 linear (4-bit weights, 16-bit activations).

TEST INFRASTRUCTURE ONLY, like ``svdq_oracle``: nothing in the product path
imports it, and it imports nothing from the HIP library.

The pages name the layer family and its configuration only ("Bringing
Nunchaku 4-bit Diffusion Inference to Diffusers", "Introducing Nunchaku
Lite": 4-bit weights with 16-bit activations for the adaptive-normalization
and modulation projections, which are memory-bound and precision-sensitive;
"Native loading in Diffusers": ``awq_w4a16`` with ``precision`` int4 and
``group_size`` 64).  The steps follow the published AWQ method
(activation-aware weight quantization: scale input channels by a power of
their mean activation magnitude before round-to-nearest, choosing the power
by a grid search on calibration activations).  Readings (each in the
design notes):

  W1  Weights: asymmetric unsigned INT4 per (output channel, group of 64
      along K): s = fp16(max(wmax - wmin, 1e-5) / 15), z = clamp(rne(-wmin /
      s), 0, 15), q = clamp(rne(w / s) + z, 0, 15); dequantized (q - z) s.
  W2  Channel scales: a_k = mean_m |X[m, k]| over the calibration rows,
      t_k = max(a_k, 1e-4)^alpha normalized by sqrt(max t * min t);
      alpha from {0, 1/20, ..., 19/20} minimizing ||X W^T - X diag(t)^-1
      Q(W diag(t))^T||_F on the calibration rows (ties: the smaller alpha).
      inv_scale = fp32(1 / t); the weight side uses t := 1 / fp64(inv_scale)
      so both sides cancel for the stored factor (as for the SVDQuant
      smoothing).
  W3  Activations: x_hat = bf16(fp32(x * inv_scale)) (16-bit operand), the
      product accumulates in fp32; Y = bf16(sum_g s_g sum_{k in g} (q - z)
      x_hat + bias).
  W4  Storage: codes [N][K/2] (low nibble = even k, unsigned), scales
      [N][K/64] fp16, zero points [N][K/64] u8.
"""
from __future__ import annotations

import numpy as np

from . import svdq_oracle as _o

__all__ = ["ALPHA_GRID", "awq_quantize", "awq_dequantize", "awq_channel_scale", "awq_prepare",
           "awq_forward", "awq_forward_bruteforce"]

GROUP = 64
ALPHA_GRID = np.arange(20) / 20.0


def awq_quantize(w_nk, group: int = GROUP):
    """W [N][K] (fp64 values) -> (q [N][K] ints 0..15, s [N][K/g] fp16 values,
    z [N][K/g] ints 0..15) (reading W1)."""
    w = np.asarray(w_nk, dtype=np.float64)
    N, K = w.shape
    wg = w.reshape(N, K // group, group)
    wmax, wmin = wg.max(axis=-1), wg.min(axis=-1)
    s = _o.fp16(np.maximum(wmax - wmin, 1e-5) / 15.0)
    z = np.clip(np.rint(-wmin / s), 0, 15)
    q = np.clip(np.rint(wg / s[..., None]) + z[..., None], 0, 15)
    return q.reshape(N, K).astype(np.int64), s, z.astype(np.int64)


def awq_dequantize(q, s, z, group: int = GROUP):
    N, K = q.shape
    return ((q.reshape(N, K // group, group) - z[..., None]) * s[..., None]).reshape(N, K)


def awq_channel_scale(x_cal, alpha: float):
    """Normalized channel scale t (fp64) for one alpha (reading W2)."""
    a = np.mean(np.abs(np.asarray(x_cal, dtype=np.float64)), axis=0)
    t = np.maximum(a, 1e-4) ** alpha
    return t / np.sqrt(t.max() * t.min())


def _stored(t):
    inv = _o.fp32(1.0 / t)
    return inv, 1.0 / inv


def awq_prepare(weight_nk, x_cal, alpha=None, group: int = GROUP):
    """Search (or take) alpha, then quantize W diag(t).  Returns a dict with
    alpha, inv_scale [K] (fp32 values), q, s, z, losses (per grid alpha)."""
    w = np.asarray(weight_nk, dtype=np.float64)
    x = np.asarray(x_cal, dtype=np.float64)
    ref = x @ w.T
    losses = None
    if alpha is None:
        losses = []
        for al in ALPHA_GRID:
            inv, t = _stored(awq_channel_scale(x, al))
            q, s, z = awq_quantize(w * t[None, :], group)
            wq = awq_dequantize(q, s, z, group) * inv[None, :]
            losses.append(float(np.sum((ref - x @ wq.T) ** 2)))
        alpha = float(ALPHA_GRID[int(np.argmin(losses))])
    inv, t = _stored(awq_channel_scale(x, alpha))
    q, s, z = awq_quantize(w * t[None, :], group)
    return dict(alpha=alpha, inv_scale=inv, q=q, s=s, z=z, losses=losses, group=group)


def awq_forward(x, prep, bias=None, out: str = "bf16"):
    """Y = bf16(x_hat @ dequant(W)^T + bias), x_hat = bf16(fp32(x * inv_scale))
    (reading W3); fp64 sums."""
    x_hat = _o.bf16(_o.fp32(np.asarray(x, dtype=np.float64) * prep["inv_scale"][None, :]))
    y = x_hat @ awq_dequantize(prep["q"], prep["s"], prep["z"], prep["group"]).T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return {"bf16": _o.bf16, "f32": _o.fp32, "f64": lambda v: v}[out](y)


def awq_forward_bruteforce(x_hat, q, s, z, group: int = GROUP):
    """Python loops over exact group sums for tiny inputs (no bias)."""
    M, K = x_hat.shape
    N = q.shape[0]
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            tot = 0.0
            for g in range(K // group):
                part = sum(float(x_hat[m, k]) * int(q[n, k] - z[n, g]) for k in range(g * group, (g + 1) * group))
                tot += part * float(s[n, g])
            out[m, n] = tot
    return out
