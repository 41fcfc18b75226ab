"""AWQ host preparation against the oracle and entry-point validation."""
import ctypes

import numpy as np
import pytest

import workloads
from oracle import awq_oracle as A

S = pytest.importorskip("w4a4_rank_corrected_svdq_amd")
from w4a4_rank_corrected_svdq_amd import _lib as L  # noqa: E402


def _pack(q):
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("alpha", [0.0, 0.35, 0.9])
def test_awq_prepare_bit_exact_given_alpha(alpha):
    wl = workloads.awq_workload(4, K=512, N=256, Mc=32, seed=46)
    po = A.awq_prepare(wl["weight"], wl["x_cal"], alpha=alpha)
    p = S.awq_prepare(wl["weight_bits"], wl["x_cal_bits"], alpha=alpha)
    np.testing.assert_array_equal(p["inv_scale"].astype(np.float64), po["inv_scale"])
    np.testing.assert_array_equal(p["w_scales"].astype(np.float64), po["s"])
    np.testing.assert_array_equal(p["w_zeros"], po["z"])
    np.testing.assert_array_equal(p["w_codes"], _pack(po["q"]))


def test_awq_prepare_search_matches_oracle():
    wl = workloads.awq_workload(4, K=512, N=256, Mc=32, seed=44)
    po = A.awq_prepare(wl["weight"], wl["x_cal"])
    p = S.awq_prepare(wl["weight_bits"], wl["x_cal_bits"])
    assert p["alpha"] == pytest.approx(po["alpha"])
    np.testing.assert_array_equal(p["w_codes"], _pack(po["q"]))


def test_awq_entry_validation_precedes_device_use():
    buf = (ctypes.c_uint8 * 4096)()
    b = (ctypes.addressof(buf) + 15) & ~15
    p = [b + 256 * i for i in range(8)]
    qa, gv = L.lib().svdq_awq_quant_act, L.lib().svdq_awq_gemv
    assert qa(p[0], p[1], 17, 128, p[2], p[3], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE       # M > 16
    assert qa(p[0], p[1], 4, 96, p[2], p[3], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert qa(None, p[1], 4, 128, p[2], p[3], None) == L.SVDQ_ERR_INVALID_ARG
    assert gv(p[0], p[1], p[2], p[3], p[4], None, 4, 48, 128, p[5], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert gv(p[0], p[1], p[2], p[3], None, None, 4, 32, 128, p[5], None) == L.SVDQ_ERR_INVALID_ARG
    assert gv(p[0], p[1], p[2], p[3], p[4], p[6] + 2, 4, 32, 128, p[5], None) == L.SVDQ_ERR_INVALID_ARG
    assert gv(p[0], p[1], p[2], p[3], p[4], None, -1, 32, 128, p[5], None) == L.SVDQ_ERR_INVALID_ARG
    with pytest.raises(S.SVDQError):
        S.awq_prepare(np.zeros((48, 128), np.uint16), np.zeros((4, 128), np.uint16))    # N % 32
