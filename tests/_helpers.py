"""Shared test helpers: layout conversions between the oracle's math layout
and the C ABI's storage layout, and the comparison bars.  No method
arithmetic lives here (the decision bands come from the oracle)."""
import numpy as np

import oracle as O


def f64_to_bf16_bits(v) -> np.ndarray:
    """Bits of values that are already exactly bf16 (asserted)."""
    v = np.asarray(v, dtype=np.float64)
    f = v.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v)
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "value is not a bf16"
    return (bits >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def oracle_prep_to_abi(p) -> dict:
    """Oracle ``prepare`` dict -> ABI arrays (w_codes [N][K/2], w_scales
    [K/64][N] f16, lora_down [r][K] bf16 bits, lora_up [N][r] bf16 bits)."""
    K, N = p["W_hat"].shape
    r = p["L1"].shape[1]
    return dict(
        smooth_inv=p["smooth_inv"].astype(np.float32),
        w_codes=O.pack_int4(p["qw"].T),
        w_scales=p["sw"].astype(np.float16),
        lora_down=f64_to_bf16_bits(p["L1"].T) if r else np.zeros((0, K), np.uint16),
        lora_up=f64_to_bf16_bits(p["L2"].T) if r else np.zeros((N, 0), np.uint16),
        rank=r, K=K, N=N,
    )


def abi_to_oracle_prep(p, group: int = 64) -> dict:
    """Library-prepared arrays (ABI storage layouts) -> the oracle's keys
    (qw [K][N] ints, sw [K/64][N], L1 [K][r], L2 [r][N], smooth_inv), so
    that the oracle's forward runs on exactly the arrays a layer holds."""
    K, N, r = int(p["K"]), int(p["N"]), int(p["rank"])
    return dict(
        smooth_inv=np.asarray(p["smooth_inv"], np.float32).astype(np.float64).reshape(K),
        qw=O.unpack_int4(np.asarray(p["w_codes"], np.uint8).reshape(N, K // 2)).T,
        sw=np.asarray(p["w_scales"], np.float16).astype(np.float64).reshape(K // group, N),
        L1=bf16_bits_to_f64(np.asarray(p["lora_down"]).reshape(r, K)).T if r else np.zeros((K, 0)),
        L2=bf16_bits_to_f64(np.asarray(p["lora_up"]).reshape(N, r)).T if r else np.zeros((0, N)),
        group=group,
    )


def ulp_bf16(v) -> np.ndarray:
    """Spacing of bf16 values at |v| (normal range)."""
    v = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -126)))
    return np.exp2(e - 7)


def check_bf16_elementwise(yg, yo, frac: float = 1e-4, atol=0.0) -> None:
    """|GPU - oracle| within one bf16 ulp of the oracle's value (plus
    ``atol``, a per-element bound on the kernel's own fp32 rounding where a
    path's arithmetic makes it larger than an ulp) for all but a ``frac``
    fraction of the elements: fp32 accumulation in another order can move a
    value across one bf16 rounding boundary, rarely two."""
    yg, yo = np.asarray(yg, np.float64), np.asarray(yo, np.float64)
    assert yg.shape == yo.shape
    d = np.maximum(np.abs(yg - yo) - atol, 0.0) / ulp_bf16(yo)
    bad = d > 1 + 1e-12
    if bad.mean() > frac:
        worst = np.argsort(d, axis=None)[::-1][:6]
        rows = [f"{np.unravel_index(i, d.shape)}: gpu {yg.flat[i]!r} oracle {yo.flat[i]!r} ({d.flat[i]:.2f} ulp)"
                for i in worst]
        raise AssertionError(f"{bad.sum()} of {bad.size} elements differ by more than one bf16 ulp:\n"
                             + "\n".join(rows))


def check_f32_elementwise(yg, yo, rel: float = 2.0 ** -14) -> None:
    """fp32 outputs: every element within rel * (|y| + rms(y)) of the
    oracle's value (the kernel's fp32 sums over at most a few hundred
    groups stay far inside this; a wrong tile or strip does not)."""
    yg, yo = np.asarray(yg, np.float64), np.asarray(yo, np.float64)
    assert yg.shape == yo.shape
    rms = np.sqrt(np.mean(yo * yo)) if yo.size else 0.0
    bad = np.abs(yg - yo) > rel * (np.abs(yo) + rms)
    assert not bad.any(), f"{bad.sum()} of {bad.size} fp32 elements outside the bound"


# The device's tanh-GELU on load (fp32, hardware exp2 and reciprocal) is
# within ~1.3e-6 relative of the oracle's fp64 tanh form after the fp32
# roundings of x_hat; the bands below allow three times that.
GELU_REL = 4e-6


def check_int4_codes_in_band(q_dev, s_dev, x_hat, rel: float = GELU_REL, group: int = 64):
    """Kernel 1's INT4 scales [M][G] and codes [M][K] against the oracle's
    decisions on x_hat under a relative band: equal wherever the oracle's
    decision is unique, one of the band's two ends elsewhere (each code
    checked against the scale the device used).  Returns the numbers of
    ambiguous scales and codes."""
    s_dev = np.asarray(s_dev, np.float64)
    s_lo, s_hi, _, _ = O.activation_decision_band(x_hat, rel, group)
    bad = (s_dev < s_lo) | (s_dev > s_hi)
    assert not bad.any(), f"{bad.sum()} scales outside the band, first at {np.argwhere(bad)[:4].tolist()}"
    _, _, q_lo, q_hi = O.activation_decision_band(x_hat, rel, group, scales=s_dev)
    q_dev = np.asarray(q_dev)
    bad = (q_dev < q_lo) | (q_dev > q_hi)
    assert not bad.any(), f"{bad.sum()} codes outside the band, first at {np.argwhere(bad)[:4].tolist()}"
    return int(np.count_nonzero(s_lo != s_hi)), int(np.count_nonzero(q_lo != q_hi))


def check_mx_codes_in_band(v_dev, e_dev, x_hat, rel: float = GELU_REL):
    """The MXFP4 counterpart: block exponents [M][K/32] and element values
    [M][K] (decoded E2M1) against the oracle's decisions under the band."""
    e_dev = np.asarray(e_dev, np.int64)
    e_lo, e_hi, _, _ = O.mx.activation_decision_band_mx(x_hat, rel)
    bad = (e_dev < e_lo) | (e_dev > e_hi)
    assert not bad.any(), f"{bad.sum()} exponents outside the band"
    _, _, q_lo, q_hi = O.mx.activation_decision_band_mx(x_hat, rel, exponents=e_dev)
    v_dev = np.asarray(v_dev, np.float64)
    bad = (v_dev < q_lo) | (v_dev > q_hi)
    assert not bad.any(), f"{bad.sum()} element values outside the band"
    return int(np.count_nonzero(e_lo != e_hi)), int(np.count_nonzero(q_lo != q_hi))
