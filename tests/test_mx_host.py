"""MXFP4 host preparation and entry-point validation (no GPU needed)."""
import ctypes

import numpy as np
import pytest

import oracle as O
import workloads
from tests._helpers import f64_to_bf16_bits

S = pytest.importorskip("w4a4_rank_corrected_svdq_amd")
from w4a4_rank_corrected_svdq_amd import _lib as L  # noqa: E402

MX = O.mx


def mx_prep_to_abi(p):
    """Oracle MX prepare dict -> ABI arrays."""
    K, N = p["W_hat"].shape
    r = p["L1"].shape[1]
    return dict(
        smooth_inv=p["smooth_inv"].astype(np.float32),
        w_codes=O.pack_int4(MX.e2m1_encode(p["qw"].T)),
        w_scales=(p["ew"].T + 127).astype(np.uint8),
        lora_down=f64_to_bf16_bits(p["L1"].T) if r else np.zeros((0, K), np.uint16),
        lora_up=f64_to_bf16_bits(p["L2"].T) if r else np.zeros((N, 0), np.uint16),
        rank=r, K=K, N=N)


@pytest.mark.parametrize("rank", [0, 16, 32])
def test_prepare_mx_bit_exact_given_factors(rank):
    """Given the oracle's bf16 factors (none at rank 0), the library's MXFP4
    residual codes and scales match the oracle's bit for bit."""
    wl = workloads.custom_workload(64, 512, 384, seed=81, n_out=6)
    Lr = wl.layers[0]
    po = MX.prepare_mx(Lr.weight, wl.act_absmax(), rank=rank)
    abi = mx_prep_to_abi(po)
    fac = (abi["lora_down"], abi["lora_up"]) if rank else None
    p = S.prepare_weights_mxfp4(Lr.weight_bits, wl.act_absmax(), rank=rank, factors=fac)
    np.testing.assert_array_equal(p["smooth_inv"], abi["smooth_inv"])
    np.testing.assert_array_equal(p["w_scales"], abi["w_scales"])
    np.testing.assert_array_equal(p["w_codes"], abi["w_codes"])


def test_prepare_mx_zero_and_tiny_blocks():
    """All-zero blocks get scale byte 0 (2^-127) and codes 0; the oracle agrees."""
    wl = workloads.custom_workload(16, 256, 64, seed=82, n_out=2)
    Lr = wl.layers[0]
    w = Lr.weight.copy()
    w[5, :] = 0.0
    w[7, 32:64] = 0.0
    bits = f64_to_bf16_bits(w)
    po = MX.prepare_mx(w, wl.act_absmax(), rank=0)
    p = S.prepare_weights_mxfp4(bits, wl.act_absmax(), rank=0)
    abi = mx_prep_to_abi(po)
    np.testing.assert_array_equal(p["w_scales"], abi["w_scales"])
    np.testing.assert_array_equal(p["w_codes"], abi["w_codes"])
    assert np.all(p["w_scales"][5] == 0) and np.all(p["w_codes"][5] == 0)
    assert p["w_scales"][7, 1] == 0


def test_prepared_bytes_mx_matches_oracle():
    assert S.prepared_bytes_mxfp4(3072, 12288, 32) == MX.prepared_bytes_mx(3072, 12288, 32)
    with pytest.raises(S.SVDQError):
        S.prepared_bytes_mxfp4(3072 + 64, 12288, 32)     # K must be a multiple of 128


def _fake(n=1):
    buf = (ctypes.c_uint8 * 4096)()
    base = (ctypes.addressof(buf) + 15) & ~15
    return buf, [base + 256 * i for i in range(n)]


def test_mx_entry_validation_precedes_device_use():
    buf, p = _fake(10)
    q = L.lib().svdq_quant_act_lora_down_mxfp4
    g = L.lib().svdq_gemm_mxfp4_lora_up
    assert q(p[0], p[1], p[2], 16, 192, 32, 0, p[3], p[4], p[5], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert q(p[0], p[1], p[2], 16, 128, 24, 0, p[3], p[4], p[5], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert q(p[0], p[1], p[2], 16, 32768 + 128, 32, 0, p[3], p[4], p[5], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert q(None, p[1], p[2], 16, 128, 32, 0, p[3], p[4], p[5], None) == L.SVDQ_ERR_INVALID_ARG
    assert q(p[0], p[1], p[2], 16, 128, 32, 5, p[3], p[4], p[5], None) == L.SVDQ_ERR_INVALID_ARG
    assert q(p[0], p[1], p[2], -1, 128, 32, 0, p[3], p[4], p[5], None) == L.SVDQ_ERR_INVALID_ARG
    assert q(p[0], p[1], p[2], 16, 128, 32, 0, p[3], p[4] + 1, p[5], None) == L.SVDQ_ERR_INVALID_ARG
    assert g(p[0], p[1], p[2], p[3], p[4], p[5], None, 16, 64, 192, 16, 0, p[6], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert g(p[0], p[1], p[2], p[3], p[4], p[5], None, 16, 60, 128, 16, 0, p[6], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert g(p[0], p[1], p[2], p[3], p[4], p[5], None, 16, 64, 128, 16, 2, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    assert g(p[0], p[1], p[2], p[3], None, None, None, 16, 64, 128, 16, 0, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    assert g(p[0], p[1], p[2], p[3], p[4], p[5], p[7] + 8, 16, 64, 128, 16, 0, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    assert g(p[0], p[1], p[2], p[3], p[4], p[5], None, 1 << 20, 64, 8192, 16, 0, p[6], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
