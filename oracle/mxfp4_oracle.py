"""CPU oracle for the 4-bit floating-point variant of the layer (MXFP4).

TEST INFRASTRUCTURE ONLY, like ``svdq_oracle``: nothing in the product path
imports it, and it imports nothing from the HIP library.

The pages offer the SVDQuant W4A4 layer in an INT4 and a 4-bit float variant
("Bringing Nunchaku 4-bit Diffusion Inference to Diffusers", "Background:
SVDQuant and Nunchaku" and the ``precision`` field of "Native loading in
Diffusers"); their float variant is a Blackwell-specific encoding.  The
4-bit float encoding that gfx950's matrix cores apply natively is the OCP
Microscaling (MX) format MXFP4, and this module takes it as the variant's
definition (reading M1):

  M1  Elements are FP4 E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa
      bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).  A block of 32 consecutive
      values along K shares one E8M0 scale 2^e (the OCP MX specification,
      v1.0, section 5: block size 32, scale = 2^(floor(log2(amax)) - 2),
      2 being the largest E2M1 exponent), e clamped to [-127, 127].
  M2  Elements are v / 2^e rounded to the nearest E2M1 value, ties to even
      mantissa; magnitudes above 6 saturate to 6.  A value that rounds to
      zero is encoded +0 (code 0).  An all-zero block has e = -127 and codes 0.
  M3  Codes are packed two per byte, low nibble = even k (as for INT4).
  M4  Everything else is the INT4 layer's: smoothing, the bf16 low-rank
      branch computed from bf16(x_hat), the fp32 x_hat = fp32(x * smooth_inv)
      on the activation side, the residual R taken against the bf16 factors,
      and Y = bf16(sum_b 2^(ex + ew) <qx, qw>_b + bf16(lora_act) L2 + bias).
"""
from __future__ import annotations

import numpy as np

from . import svdq_oracle as _o

__all__ = ["E2M1_VALUES", "e2m1_round", "e2m1_encode", "e2m1_decode", "mx_block_exponent",
           "mx_quantize", "quantize_activation_mx", "prepare_mx", "mx_product",
           "mx_product_bruteforce", "forward_mx", "prepared_bytes_mx"]

BLOCK = 32
EMAX_ELEM = 2           # largest exponent of E2M1 (6 = 1.5 * 2^2)
E2M1_MAX = 6.0
# code -> value for codes 0..7 (codes 8..15 are the negatives)
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_round(v) -> np.ndarray:
    """Nearest E2M1 value, ties to the even mantissa bit, saturating at +-6
    (reading M2).  Works on fp64 values; returns fp64."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    grid = E2M1_VALUES
    # index of the largest grid value <= a
    lo = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    glo, ghi = grid[lo], grid[hi]
    dlo, dhi = a - glo, ghi - a
    # codes 0..7: the mantissa bit is the code's low bit; ties go to the even code
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0) & (hi != lo))
    r = np.where(pick_hi, ghi, glo)
    r = np.where(a >= E2M1_MAX, E2M1_MAX, r)
    return np.where(v < 0, -r, r) + 0.0  # -0 -> +0


def e2m1_encode(vals) -> np.ndarray:
    """E2M1 values (already on the grid) -> codes 0..15 (zero -> 0)."""
    vals = np.asarray(vals, dtype=np.float64)
    mag = np.abs(vals)
    idx = np.searchsorted(E2M1_VALUES, mag)
    if not np.all(E2M1_VALUES[np.minimum(idx, 7)] == mag):
        raise ValueError("value not on the E2M1 grid")
    return np.where((vals < 0) & (mag > 0), idx + 8, idx).astype(np.int64)


def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    v = E2M1_VALUES[c & 7]
    return np.where(c & 8, -v, v)


def mx_block_exponent(amax) -> np.ndarray:
    """floor(log2(amax)) - 2, clamped to [-127, 127]; -127 for amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    m, ex = np.frexp(amax)          # amax = m * 2^ex, m in [0.5, 1): floor(log2) = ex - 1
    e = (ex - 1) - EMAX_ELEM
    e = np.where(amax == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def mx_quantize(v, axis: int):
    """MXFP4 quantization of fp64 values in blocks of 32 along ``axis``.
    Returns (element values on the E2M1 grid, same shape as v; exponents e
    with that axis reduced by 32)."""
    v = np.asarray(v, dtype=np.float64)
    vm = np.moveaxis(v, axis, -1)
    shp = vm.shape
    if shp[-1] % BLOCK:
        raise ValueError("length along the block axis must be a multiple of 32")
    vb = vm.reshape(shp[:-1] + (shp[-1] // BLOCK, BLOCK))
    e = mx_block_exponent(np.abs(vb).max(axis=-1))
    q = e2m1_round(vb * np.ldexp(1.0, -e)[..., None])
    q = np.moveaxis(q.reshape(shp), -1, axis)
    return q, np.moveaxis(e, -1, axis)


def quantize_activation_mx(x, smooth_inv, act: str = "none"):
    """Activation side with the GPU's fp32 rounding points (reading M4):
    x_hat = fp32(act(x) * smooth_inv); amax over each block of 32 is exact;
    x_hat * 2^-e is exact (a power-of-two scaling; values small enough to
    lose bits round to 0 in E2M1 either way).  Returns (element values [M x K],
    exponents [M x K/32], x_hat)."""
    x = np.asarray(x, dtype=np.float64)
    if act == "gelu_tanh":
        x = _o.fp32(_o.gelu_tanh(x))
    x_hat = _o.fp32(x * np.asarray(smooth_inv, dtype=np.float64)[None, :])
    q, e = mx_quantize(x_hat, axis=1)
    return q, e, x_hat


def activation_decision_band_mx(x_hat, rel: float, exponents=None):
    """The activation side's MXFP4 decisions (readings M2, M4) when every
    value of x_hat may be off by a relative ``rel`` (another correct fp32
    evaluation of the input function, such as the tanh-GELU on load).  The
    block exponent and the E2M1 rounding are monotone in what they round, so
    each decision lies between its results at the two ends of the band:
      exponents (e_lo, e_hi) [M x K/32] from the block absmax times (1 -+ rel);
      element values (q_lo, q_hi) [M x K] from x_hat 2^-e -+ |.| rel, with e
        the exponents actually used (``exponents``; e_lo when None).
    With rel = 0 this is quantize_activation_mx's quantizer exactly."""
    x_hat = np.asarray(x_hat, dtype=np.float64)
    M, K = x_hat.shape
    xb = x_hat.reshape(M, K // BLOCK, BLOCK)
    amax = np.abs(xb).max(axis=-1)
    e_lo = mx_block_exponent(amax * (1.0 - rel))
    e_hi = mx_block_exponent(amax * (1.0 + rel))
    e = e_lo if exponents is None else np.asarray(exponents, dtype=np.int64).reshape(e_lo.shape)
    v = xb * np.ldexp(1.0, -e)[..., None]
    q_lo = e2m1_round(v - np.abs(v) * rel).reshape(M, K)
    q_hi = e2m1_round(v + np.abs(v) * rel).reshape(M, K)
    return e_lo, e_hi, q_lo, q_hi


def prepare_mx(weight_nk, act_absmax, rank: int, alpha: float = 0.5, factors=None):
    """Preparation as ``svdq_oracle.prepare`` (smoothing, split, residual) with
    the residual quantized to MXFP4 along K per output channel."""
    p = _o.prepare(weight_nk, act_absmax, rank, alpha=alpha, factors=factors, quantize=False)
    p["qw"], p["ew"] = mx_quantize(p["R"], axis=0)      # [K x N], [K/32 x N]
    p["block"] = BLOCK
    return p


def prepared_bytes_mx(K: int, N: int, rank: int) -> int:
    """Packed E2M1 codes, one E8M0 byte per block, bf16 factors, fp32 smooth_inv."""
    return N * K // 2 + (K // BLOCK) * N + 2 * rank * (K + N) + 4 * K


def mx_product(qx, ex, qw, ew) -> np.ndarray:
    """sum_b 2^(ex[m,b] + ew[b,n]) * sum_{k in b} qx[m,k] qw[k,n] in fp64
    (each block sum is a multiple of 1/4 below 2^11: exact)."""
    M, K = qx.shape
    acc = np.zeros((M, qw.shape[1]))
    for b in range(K // BLOCK):
        sl = slice(b * BLOCK, (b + 1) * BLOCK)
        acc += np.ldexp(1.0, ex[:, b])[:, None] * np.ldexp(1.0, ew[b, :])[None, :] * (qx[:, sl] @ qw[sl, :])
    return acc


def mx_product_bruteforce(qx, ex, qw, ew):
    """Python-int loops over exact rationals (quarter units) for tiny inputs."""
    from fractions import Fraction
    M, K = qx.shape
    N = qw.shape[1]
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for b in range(K // BLOCK):
                s = sum(int(qx[m, k] * 2) * int(qw[k, n] * 2) for k in range(b * BLOCK, (b + 1) * BLOCK))
                tot += Fraction(s, 4) * Fraction(2) ** int(ex[m, b] + ew[b, n])
            out[m, n] = float(tot)
    return out


def forward_mx(x, prep, bias=None, act: str = "none", out: str = "bf16", return_parts: bool = False):
    """Y = MXFP4(X_hat) MXFP4(R) + bf16(bf16(X_hat) L1) L2 + bias (reading M4)."""
    qx, ex, x_hat = quantize_activation_mx(x, prep["smooth_inv"], act)
    acc = mx_product(qx, ex, prep["qw"], prep["ew"])
    rank = prep["L1"].shape[1]
    la = _o.lora_down(x_hat, prep["L1"]) if rank else np.zeros((x_hat.shape[0], 0))
    y = acc + (_o.bf16(la) @ prep["L2"] if rank else 0.0)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    Y = {"bf16": _o.bf16, "f32": _o.fp32, "f64": lambda v: v}[out](y)
    if return_parts:
        return Y, dict(qx=qx, ex=ex, x_hat=x_hat, lora_act=la, acc=acc, y=y)
    return Y
