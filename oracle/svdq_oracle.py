"""CPU oracle for the SVDQuant W4A4 linear with a rank-r 16-bit correction.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``w4a4_rank_corrected_svdq_amd``) and imports nothing from it.

Plain numpy, fp64 unless a step's storage format fixes the precision.  The
steps follow the pages in their order:

* svdq-int4-flux.1-depth-dev model card, "Quantization Method -- SVDQuant":
  stage 1 (activations and weights both carry outliers), stage 2 (outliers
  move from the activation into the weight: X_hat = X diag(lambda)^-1,
  W_hat = diag(lambda) W), stage 3 (W_hat is split by SVD into a 16-bit
  low-rank branch L1 L2 plus a residual R).
* "Bringing Nunchaku 4-bit Diffusion Inference to Diffusers",
  "Background: SVDQuant and Nunchaku": the residual is quantized to 4 bits and
  the main product runs with 4-bit weights and activations (W4A4); the
  low-rank branch stays at 16 bits.
* model card, "Nunchaku Engine Design": the down projection X_hat L1 reads the
  same 16-bit input as the activation quantizer, and the up projection
  (X_hat L1) L2 adds into the same 16-bit output as the 4-bit product.
* Rank 32 is the pages' branch rank (model card, "Nunchaku Engine Design";
  "Native loading in Diffusers" config).  Group size 64 along K and the
  symmetric INT4 encoding with fp16 scales are the readings listed below.

Readings where the pages are silent (each also listed in the design doc):
  R1  lambda_j = max(a_j,eps)^alpha / max(w_j,eps)^(1-alpha), alpha = 0.5,
      eps = 1e-5, a = calibration absmax of X[:, j], w = max_n |W[j, n]|
      (SmoothQuant-style; the pages give no formula).  smooth_inv = fp32(1/lambda);
      the weight side uses lambda := 1/fp64(smooth_inv) so that both sides
      cancel for the stored factor.
  R2  Sigma is folded into L1 (L1 = U_r Sigma_r, L2 = V_r^T); both rounded to
      bf16 (the pages' 16-bit type; the Diffusers config names bfloat16).
  R3  R = W_hat - bf16(L1) bf16(L2): the residual is taken against the factors
      that actually run.
  R4  INT4 symmetric, group 64 along K: per (group, output channel) for R, per
      (token, group) for X; scale s = fp16(absmax / 7) (round to nearest even),
      code q = clamp(rne(v / s), -8, 7); an all-zero group has s = 0, q = 0.
  R5  GPU arithmetic for the activation quantizer is fp32: x_hat =
      f32(x * smooth_inv), s32 = f32(a / 7), s = fp16(s32),
      rcp = f32(1 / f32(s)) (0 if s == 0), q = clamp(rne(f32(x_hat * rcp))).
  R6  The down projection consumes bf16(x_hat); lora_act is stored fp32 and
      rounded to bf16 where it meets L2.
  R7  Packing: two codes per byte, low nibble = even k, two's complement.
  R8  Output Y = bf16(acc + bf16(lora_act) L2 + bias), round to nearest even.
  R9  Optional tanh-GELU (textbook tanh form) on the bf16 input of the
      quantizer, in fp32, before smoothing (MLP pair chain).
  R11 Fused QKV operator (the Diffusers page, "Quantizing models with
      structural rewrites": the fused operator consumes the QKV projection,
      the Q/K normalization and the rotary embeddings together): the
      projection's output is [Q | K | V] along N, each H heads of 128; Q and K
      heads get RMSNorm over the head (eps 1e-6, a learnable weight per
      element) and then the rotary embedding on adjacent pairs (2i, 2i+1)
      with per-token angle tables; V is left as projected.  Both act on the
      fp32 projection before the single bf16 rounding of the output.
  R10 The unfused comparison path (``forward_unfused``) stores the 4-bit
      GEMM's output plus bias as bf16 before the up projection adds to it,
      and rounds to bf16 again: the 16-bit output is written twice.
  G1  The tanh-GELU of R9 may be evaluated anywhere within a relative 4e-6 of
      the exact function; where that can move a group's scale or a code
      across its rounding boundary, both results are valid
      (``activation_decision_band`` states the band).

Emulating one fp32 operation by computing it in fp64 and rounding once to
fp32 gives the correctly rounded fp32 result for +, -, *, / and sqrt, since
53 >= 2*24 + 2; the oracle uses this for the fp32 steps of R5.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "round_to_bits", "bf16", "fp16", "fp32",
    "smoothing_factors", "smooth_weight", "low_rank_split", "quantize_groups",
    "quantize_weight_residual", "prepare", "gelu_tanh", "quantize_activation",
    "activation_decision_band",
    "pack_int4", "unpack_int4", "lora_down", "w4a4_product",
    "w4a4_product_bruteforce", "forward", "forward_unfused", "reference_fp64", "rel_fro",
    "rms_norm", "rope", "forward_qkv", "forward_mlp_chain",
    "prepared_bytes",
]

INT4_MIN, INT4_MAX = -8, 7
QMAX = 7.0  # symmetric range: absmax maps to +-7


# --------------------------------------------------------------------------
# Rounding to storage formats (round to nearest, ties to even).
# --------------------------------------------------------------------------
def round_to_bits(x, mant_bits: int, emin: int, emax: int) -> np.ndarray:
    """Round fp64 values to a binary format with ``mant_bits`` significand bits
    (implicit bit included), minimum normal exponent ``emin`` and maximum
    exponent ``emax``; ties to even; overflow -> +-inf; subnormals kept."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    _, e = np.frexp(np.abs(xf))          # |x| = m * 2^e, m in [0.5, 1)
    e = np.maximum(e - 1, emin)            # exponent of the leading bit
    quantum = np.ldexp(1.0, e - (mant_bits - 1))
    r = np.round(xf / quantum) * quantum   # np.round: ties to even; division exact
    maxval = np.ldexp(2.0 - np.ldexp(1.0, 1 - mant_bits), emax)
    r = np.where(np.abs(r) > maxval, np.copysign(np.inf, r), r)
    out[finite] = r
    return out


def bf16(x):
    return round_to_bits(x, 8, -126, 127)


def fp16(x):
    return round_to_bits(x, 11, -14, 15)


def fp32(x):
    return round_to_bits(x, 24, -126, 127)


# --------------------------------------------------------------------------
# Stage 2: smoothing (outliers move from activations into weights).
# --------------------------------------------------------------------------
def smoothing_factors(act_absmax, weight_nk, alpha: float = 0.5, eps: float = 1e-5):
    """Per-input-channel smoothing (reading R1).

    act_absmax: [K] float32 calibration maxima of |X[:, j]|.
    weight_nk:  [N][K] weight values (torch.nn.Linear layout).
    Returns (smooth_inv [K] fp32 values as fp64, lam [K] fp64) where
    lam = 1 / smooth_inv exactly as the weight side must use it.
    """
    a = np.maximum(np.asarray(act_absmax, dtype=np.float64), eps)
    w = np.maximum(np.abs(np.asarray(weight_nk, dtype=np.float64)).max(axis=0), eps)
    if alpha == 0.5:
        lam0 = np.sqrt(a / w)
    else:
        lam0 = a ** alpha / w ** (1.0 - alpha)
    smooth_inv = fp32(1.0 / lam0)
    lam = 1.0 / smooth_inv
    return smooth_inv, lam


def smooth_weight(weight_nk, lam) -> np.ndarray:
    """W_hat = diag(lambda) W with W the [K x N] math-layout weight."""
    W = np.asarray(weight_nk, dtype=np.float64).T
    return np.ascontiguousarray(lam[:, None] * W)


# --------------------------------------------------------------------------
# Stage 3: low-rank split by SVD.
# --------------------------------------------------------------------------
def low_rank_split(W_hat, rank: int, round_factors: bool = True):
    """Top-``rank`` SVD of W_hat [K x N]: L1 = U_r Sigma_r [K x r],
    L2 = V_r^T [r x N] (reading R2).  LAPACK via numpy."""
    K, N = W_hat.shape
    if rank == 0:
        return np.zeros((K, 0)), np.zeros((0, N)), np.zeros(0)
    U, S, Vt = np.linalg.svd(W_hat, full_matrices=False)
    L1 = U[:, :rank] * S[None, :rank]
    L2 = Vt[:rank, :].copy()
    if round_factors:
        L1, L2 = bf16(L1), bf16(L2)
    return L1, L2, S


# --------------------------------------------------------------------------
# 4-bit symmetric group quantization (reading R4).
# --------------------------------------------------------------------------
def quantize_groups(v, group: int, axis: int):
    """Quantize fp64 values ``v`` in groups of ``group`` along ``axis``.
    Returns (codes int64 same shape as v, scales fp64 with that axis reduced
    by ``group``).  Scale = fp16(absmax / 7) rounded directly from fp64."""
    v = np.asarray(v, dtype=np.float64)
    vm = np.moveaxis(v, axis, -1)
    shp = vm.shape
    G = shp[-1] // group
    vg = vm.reshape(shp[:-1] + (G, group))
    a = np.abs(vg).max(axis=-1)
    s = fp16(a / QMAX)
    if not np.all(np.isfinite(s)):
        raise OverflowError("group scale overflows fp16")
    safe = np.where(s == 0, 1.0, s)
    q = np.where(s[..., None] == 0, 0.0, np.rint(vg / safe[..., None]))
    q = np.clip(q, INT4_MIN, INT4_MAX).astype(np.int64)
    q = np.moveaxis(q.reshape(shp), -1, axis)
    s = np.moveaxis(s, -1, axis)
    return q, s


def quantize_weight_residual(R, group: int = 64):
    """R [K x N] -> codes q_w [K x N], scales s_w [K/group x N]."""
    return quantize_groups(R, group, axis=0)


def prepare(weight_nk, act_absmax, rank: int, group: int = 64, alpha: float = 0.5,
            round_factors: bool = True, quantize: bool = True, factors=None):
    """Host-side preparation of one layer (stages 2-3 and the 4-bit residual).

    ``factors`` = (L1, L2) skips the SVD and uses the given factors.
    Returns a dict with smooth_inv, lam, W_hat, L1, L2, R, qw, sw, sigma.
    """
    smooth_inv, lam = smoothing_factors(act_absmax, weight_nk, alpha)
    W_hat = smooth_weight(weight_nk, lam)
    if factors is None:
        L1, L2, S = low_rank_split(W_hat, rank, round_factors)
    else:
        L1, L2 = (np.asarray(f, dtype=np.float64) for f in factors)
        S = None
    R = W_hat - L1 @ L2 if rank else W_hat.copy()
    out = dict(smooth_inv=smooth_inv, lam=lam, W_hat=W_hat, L1=L1, L2=L2, R=R,
               sigma=S, rank=rank, group=group)
    if quantize:
        out["qw"], out["sw"] = quantize_weight_residual(R, group)
    return out


def prepared_bytes(K: int, N: int, rank: int, group: int = 64) -> int:
    """Bytes of one prepared layer: packed codes, fp16 scales, bf16 L1 and L2,
    fp32 smooth_inv."""
    return N * K // 2 + 2 * (K // group) * N + 2 * rank * (K + N) + 4 * K


# --------------------------------------------------------------------------
# Activation side (GPU arithmetic, reading R5).
# --------------------------------------------------------------------------
def gelu_tanh(x):
    """Textbook tanh-form GELU in fp64 (reading R9)."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def quantize_activation(x, smooth_inv, group: int = 64, act: str = "none",
                        semantics: str = "gpu"):
    """Smooth + per-(token, group) symmetric INT4 quantization.

    x: [M x K] bf16 values (fp64 container).  Returns (q_x [M x K] int64,
    s_x [M x K/group] fp16 values, x_hat [M x K] values fed to the quantizer).
    semantics='gpu' mirrors the fp32 rounding points of reading R5;
    semantics='fp64' keeps x_hat and the division in fp64 (accuracy studies).
    """
    x = np.asarray(x, dtype=np.float64)
    if act == "gelu_tanh":
        x = fp32(gelu_tanh(x)) if semantics == "gpu" else gelu_tanh(x)
    elif act != "none":
        raise ValueError(act)
    M, K = x.shape
    G = K // group
    if semantics == "fp64":
        x_hat = x * np.asarray(smooth_inv, dtype=np.float64)[None, :]
        q, s = quantize_groups(x_hat, group, axis=1)
        return q, s, x_hat
    x_hat = fp32(x * np.asarray(smooth_inv, dtype=np.float64)[None, :])
    xg = x_hat.reshape(M, G, group)
    a = np.abs(xg).max(axis=-1)
    s32 = fp32(a / QMAX)
    s = fp16(s32)
    with np.errstate(divide="ignore"):
        rcp = np.where(s == 0, 0.0, fp32(1.0 / np.where(s == 0, 1.0, s)))
    rcp = np.where(np.isinf(s), 0.0, rcp)
    q = np.clip(np.rint(fp32(xg * rcp[..., None])), INT4_MIN, INT4_MAX).astype(np.int64)
    return q.reshape(M, K), s, x_hat


def activation_decision_band(x_hat, rel: float, group: int = 64, scales=None):
    """The activation quantizer's decisions (reading R5) when every value of
    x_hat may be off by a relative ``rel``: what another correct evaluation
    of the same input function (the tanh-GELU on load, evaluated in fp32 to
    ~1e-6 relative) may legitimately produce.

    Both decisions are monotone in the value they round, so each lies between
    its results at the two ends of the band:
      scales (s_lo, s_hi) [M x G]: fp16(fp32(a (1 -+ rel) / 7)), a the group absmax;
      codes (q_lo, q_hi) [M x K]: clamp(rne(fp32(v -+ |v| rel)), -8, 7), with
        v = x_hat * fp32(1 / s) for the scales s actually used (``scales``
        [M x G]; the band's own lower scales when None).
    Where lo == hi the decision is unique; elsewhere either end is valid.
    With rel = 0 this is quantize_activation's quantizer exactly."""
    x_hat = np.asarray(x_hat, dtype=np.float64)
    M, K = x_hat.shape
    G = K // group
    xg = x_hat.reshape(M, G, group)
    a = np.abs(xg).max(axis=-1)
    s_lo = fp16(fp32(a * (1.0 - rel) / QMAX))
    s_hi = fp16(fp32(a * (1.0 + rel) / QMAX))
    s = s_lo if scales is None else np.asarray(scales, dtype=np.float64).reshape(M, G)
    with np.errstate(divide="ignore"):
        rcp = np.where(s == 0, 0.0, fp32(1.0 / np.where(s == 0, 1.0, s)))
    v = xg * rcp[..., None]
    q_lo = np.clip(np.rint(fp32(v - np.abs(v) * rel)), INT4_MIN, INT4_MAX).astype(np.int64)
    q_hi = np.clip(np.rint(fp32(v + np.abs(v) * rel)), INT4_MIN, INT4_MAX).astype(np.int64)
    return s_lo, s_hi, q_lo.reshape(M, K), q_hi.reshape(M, K)


def pack_int4(q) -> np.ndarray:
    """[rows x K] codes in [-8, 7] -> [rows x K/2] uint8, low nibble = even k."""
    q = np.asarray(q, dtype=np.int64)
    lo = q[:, 0::2] & 0xF
    hi = q[:, 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.int64)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    q = np.empty((b.shape[0], b.shape[1] * 2), dtype=np.int64)
    q[:, 0::2], q[:, 1::2] = lo, hi
    return np.where(q >= 8, q - 16, q)


# --------------------------------------------------------------------------
# Products.
# --------------------------------------------------------------------------
def lora_down(x_hat, L1) -> np.ndarray:
    """lora_act = fp32( sum_k bf16(x_hat) L1 ) with fp64 accumulation (R6)."""
    return fp32(bf16(x_hat) @ np.asarray(L1, dtype=np.float64))


def w4a4_product(qx, sx, qw, sw, group: int = 64) -> np.ndarray:
    """acc[m, n] = sum_g s_x[m, g] s_w[g, n] P_g[m, n] with
    P_g = sum_{k in g} q_x[m, k] q_w[k, n] exact (integer-valued fp64 BLAS:
    |P_g| <= 4096 and every partial sum is an integer below 2^53)."""
    qx = np.asarray(qx, dtype=np.float64)
    qw = np.asarray(qw, dtype=np.float64)
    M, K = qx.shape
    N = qw.shape[1]
    acc = np.zeros((M, N))
    for g in range(K // group):
        sl = slice(g * group, (g + 1) * group)
        P = qx[:, sl] @ qw[sl, :]
        acc += (sx[:, g][:, None] * sw[g, :][None, :]) * P
    return acc


def w4a4_product_bruteforce(qx, qw, group: int = 64):
    """Per-group integer dot products with Python ints: list over g of
    [M][N] nested lists.  Tiny shapes only."""
    M, K = len(qx), len(qx[0])
    N = len(qw[0])
    out = []
    for g in range(K // group):
        Pg = [[0] * N for _ in range(M)]
        for m in range(M):
            for n in range(N):
                t = 0
                for k in range(g * group, (g + 1) * group):
                    t += int(qx[m][k]) * int(qw[k][n])
                Pg[m][n] = t
        out.append(Pg)
    return out


def forward(x, prep, bias=None, act: str = "none", out: str = "bf16",
            semantics: str = "gpu", quantize: bool = True, return_parts: bool = False):
    """Y = Q4(X_hat) Q4(R) + bf16(bf16(X_hat) L1) L2 + bias.

    x: [M x K] bf16 values.  prep: dict from ``prepare`` (or the same keys).
    out='bf16' rounds the fp64 result to bf16 (R8); 'f32' rounds to fp32;
    'f64' returns the fp64 value.  quantize=False uses X_hat and R unquantized.
    """
    x = np.asarray(x, dtype=np.float64)
    group = prep["group"]
    rank = prep["L1"].shape[1]
    if quantize:
        qx, sx, x_hat = quantize_activation(x, prep["smooth_inv"], group, act, semantics)
        acc = w4a4_product(qx, sx, prep["qw"], prep["sw"], group)
    else:
        xa = gelu_tanh(x) if act == "gelu_tanh" else x
        x_hat = xa * prep["smooth_inv"][None, :]
        acc = x_hat @ prep["R"]
        qx = sx = None
    if rank:
        if quantize:
            la = lora_down(x_hat, prep["L1"])
            y = acc + bf16(la) @ prep["L2"]
        else:
            la = x_hat @ prep["L1"]
            y = acc + la @ prep["L2"]
    else:
        la = np.zeros((x.shape[0], 0))
        y = acc
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    if out == "bf16":
        Y = bf16(y)
    elif out == "f32":
        Y = fp32(y)
    elif out == "f64":
        Y = y
    else:
        raise ValueError(out)
    if return_parts:
        return Y, dict(qx=qx, sx=sx, x_hat=x_hat, lora_act=la, acc=acc, y=y)
    return Y


def forward_unfused(x, prep, bias=None, act: str = "none", semantics: str = "gpu") -> np.ndarray:
    """The layer with its low-rank branch run as two separate passes, the
    naive arrangement the model card's "Nunchaku Engine Design" (a)
    measures against the fused one: the 4-bit GEMM writes its 16-bit output
    (bias included), a separate down projection re-reads X, and a separate
    up projection reads that output back, adds bf16(lora_act) L2 and writes
    it again.  The result differs from ``forward`` only by the extra bf16
    rounding of the intermediate output (reading R10).  Returns bf16 values.
    """
    x = np.asarray(x, dtype=np.float64)
    group = prep["group"]
    qx, sx, x_hat = quantize_activation(x, prep["smooth_inv"], group, act, semantics)
    y0 = w4a4_product(qx, sx, prep["qw"], prep["sw"], group)
    if bias is not None:
        y0 = y0 + np.asarray(bias, dtype=np.float64)[None, :]
    y0 = bf16(y0)
    if prep["L1"].shape[1] == 0:
        return y0
    la = lora_down(x_hat, prep["L1"])
    return bf16(y0 + bf16(la) @ prep["L2"])


def forward_mlp_chain(x, prep_up, prep_down, bias_up=None, bias_down=None, slice_cols: int = 256,
                      return_parts: bool = False):
    """The MLP pair as one chain ("Introducing Nunchaku Lite": the fused
    GELU/MLP kernels of the original engine; reading C1): the up layer's
    output Y_up = forward(x, up) rounded to bf16 once, tanh-GELU and the down
    layer's smoothing and per-(token, group) INT4 quantizer applied to it,
    the down layer's down projection bf16(x_hat) L1 formed as a sum of
    per-column-slice partials of ``slice_cols`` columns of Y_up, each rounded
    to fp32 and added in slice order in fp32 (the chain's one rounding point
    beyond the two-layer composition), then the down layer's 4-bit product,
    up projection and bias.  With one slice it is the composition
    forward(forward(x, up), down, act="gelu_tanh")."""
    y_up = forward(x, prep_up, bias=bias_up)                           # bf16 values
    group = prep_down["group"]
    qx, sx, x_hat = quantize_activation(y_up, prep_down["smooth_inv"], group, act="gelu_tanh")
    L1 = np.asarray(prep_down["L1"], dtype=np.float64)
    K = y_up.shape[1]
    la = None
    if L1.shape[1]:
        la = np.zeros((y_up.shape[0], L1.shape[1]))
        for c0 in range(0, K, slice_cols):
            part = fp32(bf16(x_hat[:, c0:c0 + slice_cols]) @ L1[c0:c0 + slice_cols])
            la = fp32(la + part)
    acc = w4a4_product(qx, sx, prep_down["qw"], prep_down["sw"], group)
    y = acc + (bf16(la) @ prep_down["L2"] if la is not None else 0.0)
    if bias_down is not None:
        y = y + np.asarray(bias_down, dtype=np.float64)[None, :]
    Y = bf16(y)
    if return_parts:
        return Y, dict(y_up=y_up, qx=qx, sx=sx, x_hat=x_hat,
                       lora_act=la if la is not None else np.zeros((y_up.shape[0], 0)))
    return Y


def rms_norm(v, g, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm over the last axis: v / sqrt(mean(v^2) + eps) * g (fp64)."""
    v = np.asarray(v, dtype=np.float64)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps) * np.asarray(g, dtype=np.float64)


def rope(v, cos, sin) -> np.ndarray:
    """Rotary embedding on adjacent pairs of the last axis: pair i of a row
    turns by the angle whose cosine and sine are cos[row, i], sin[row, i].
    v: [M, H, D]; cos, sin: [M, D/2] (shared by the heads)."""
    v = np.asarray(v, dtype=np.float64)
    c = np.asarray(cos, dtype=np.float64)[:, None, :]
    s = np.asarray(sin, dtype=np.float64)[:, None, :]
    v0, v1 = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = v0 * c - v1 * s
    out[..., 1::2] = v1 * c + v0 * s
    return out


def forward_qkv(x, prep, bias, norm_q, norm_k, cos=None, sin=None, eps: float = 1e-6,
                head_dim: int = 128, act: str = "none", out: str = "bf16") -> np.ndarray:
    """The fused QKV operator (reading R11): projection (as ``forward``, kept
    in fp64), per-head RMSNorm of Q and K, rotary embedding of Q and K, one
    rounding of the whole [M][3 H D] output."""
    y = forward(x, prep, bias=bias, act=act, out="f64")
    M, N = y.shape
    if N % (3 * head_dim):
        raise ValueError("N must be 3 * heads * head_dim")
    HD = N // 3
    H = HD // head_dim
    res = y.copy()
    for part, g in ((0, norm_q), (1, norm_k)):
        t = y[:, part * HD:(part + 1) * HD].reshape(M, H, head_dim)
        t = rms_norm(t, g, eps)
        if cos is not None:
            t = rope(t, cos, sin)
        res[:, part * HD:(part + 1) * HD] = t.reshape(M, HD)
    return {"bf16": bf16, "f32": fp32, "f64": lambda v: v}[out](res)


def reference_fp64(x, weight_nk, bias=None, act: str = "none") -> np.ndarray:
    """The unquantized layer Y* = act(X) W (+ bias) in fp64."""
    x = np.asarray(x, dtype=np.float64)
    if act == "gelu_tanh":
        x = gelu_tanh(x)
    y = x @ np.asarray(weight_nk, dtype=np.float64).T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def rel_fro(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    d = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (d if d else 1.0))
