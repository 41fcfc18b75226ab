"""The 6-bit operand container of the INT4 layer (host side, no GPU).

The integer codes of the layer (-8 .. 7) travel to the 6-bit MFMA as E3M2
values in the fragment layout declared in include/svdq.h.  These tests pin a
decoder written here from the E3M2 definition (sign bit 5, exponent bits
4..2 with bias 3, two mantissa bits; exponent 0 is subnormal), then check
the library's host packer through it.
"""
import numpy as np
import pytest

import oracle as O
from tests._fp6 import decode_fp6, e3m2_value

S = pytest.importorskip("w4a4_rank_corrected_svdq_amd")
from w4a4_rank_corrected_svdq_amd import _lib as L  # noqa: E402


def test_e3m2_decoder_against_definition():
    # hand-worked values of the format: +-0, the subnormals, the integers
    # the layer uses, the largest value 1.75 * 2^4
    cases = {0x00: 0.0, 0x20: -0.0, 0x01: 0.0625, 0x02: 0.125, 0x03: 0.1875,
             0x04: 0.25, 0x0C: 1.0, 0x10: 2.0, 0x12: 3.0, 0x14: 4.0, 0x15: 5.0,
             0x16: 6.0, 0x17: 7.0, 0x18: 8.0, 0x2C: -1.0, 0x37: -7.0, 0x38: -8.0,
             0x1F: 28.0, 0x3F: -28.0, 0x0D: 1.25, 0x0E: 1.5, 0x0F: 1.75}
    for c, v in cases.items():
        got = e3m2_value(np.array([c]))[0]
        assert got == v and np.signbit(got) == np.signbit(v), (hex(c), got, v)
    # every integer -8 .. 8 has exactly one code (two for 0)
    vals = e3m2_value(np.arange(64))
    for q in range(-8, 9):
        n = np.count_nonzero(vals == q)
        assert n == (2 if q == 0 else 1), q


@pytest.mark.parametrize("layout", [L.SVDQ_FP6_ACTIVATIONS, L.SVDQ_FP6_WEIGHTS])
@pytest.mark.parametrize("rows,K", [(1, 64), (31, 128), (32, 64), (33, 192), (200, 320), (257, 64), (130, 128)])
def test_pack_roundtrip(layout, rows, K):
    rng = np.random.default_rng(rows * 31 + K + layout)
    q = rng.integers(-8, 8, (rows, K))
    q[0, :] = -8
    q[-1, ::3] = 7
    buf = S.pack_fp6_operand(O.pack_int4(q), layout)
    rb = (rows + 31) // 32 if layout == L.SVDQ_FP6_ACTIVATIONS else 4 * ((rows + 127) // 128)
    assert buf.shape == (K // 64, rb, 1536)
    assert buf.nbytes == S.fp6_operand_bytes(rows, K, layout)
    dec, pad = decode_fp6(buf, rows, K, layout)
    np.testing.assert_array_equal(dec, q)
    # slots past the last row are +0 (byte value 0), zeros are +0 too
    assert np.all(pad == 0)


def test_pack_zero_codes_are_positive_zero():
    q = np.zeros((40, 128), np.int64)
    buf = S.pack_fp6_operand(O.pack_int4(q), L.SVDQ_FP6_WEIGHTS)
    assert not buf.any()


def test_operand_bytes_and_errors():
    assert S.fp6_operand_bytes(4096, 3072, L.SVDQ_FP6_ACTIVATIONS) == 48 * 128 * 1536
    assert S.fp6_operand_bytes(12288, 3072, L.SVDQ_FP6_WEIGHTS) == 48 * 384 * 1536
    assert S.fp6_operand_bytes(100, 3072, L.SVDQ_FP6_WEIGHTS) == 48 * 4 * 1536
    lib = L.lib()
    import ctypes
    out = ctypes.c_size_t(0)
    assert lib.svdq_fp6_operand_bytes(10, 100, 0, ctypes.byref(out)) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert lib.svdq_fp6_operand_bytes(10, 64, 2, ctypes.byref(out)) == L.SVDQ_ERR_INVALID_ARG
    assert lib.svdq_fp6_operand_bytes(-1, 64, 0, ctypes.byref(out)) == L.SVDQ_ERR_INVALID_ARG
    assert lib.svdq_fp6_operand_bytes(10, 64, 0, None) == L.SVDQ_ERR_INVALID_ARG
    assert lib.svdq_pack_fp6_operand(None, 10, 64, 0, None) == L.SVDQ_ERR_INVALID_ARG
