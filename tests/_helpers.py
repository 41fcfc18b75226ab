"""Shared test helpers: layout conversions between the oracle's math layout
and the C ABI's storage layout.  No method arithmetic lives here."""
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
