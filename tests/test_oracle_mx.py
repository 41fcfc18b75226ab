"""Pins for the MXFP4 oracle: the E2M1 table against its bit definition,
hand-worked rounding and block fixtures, brute force, the dequantized
definition and the error story."""
import os

import numpy as np
import pytest

import oracle as O
import workloads

MX = O.mx
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append([p.strip() for p in line.split("|")])
    return out


def test_e2m1_table_golden_and_bit_definition():
    rows = _rows("e2m1_codes.txt")
    assert len(rows) == 16
    for code, bits, val in rows:
        c = int(code)
        assert int(bits, 2) == c
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        closed = (m * 0.5) if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        closed = -closed if s else closed
        assert closed == float(val)
        assert MX.e2m1_decode(c) == float(val)
    # encode is the inverse on the grid (zero always encodes as code 0)
    codes = np.arange(16)
    vals = MX.e2m1_decode(codes)
    enc = MX.e2m1_encode(vals)
    np.testing.assert_array_equal(enc, np.where(codes == 8, 0, codes))


def test_e2m1_rounding_golden():
    for inp, exp, _ in _rows("e2m1_rounding.txt"):
        got = float(MX.e2m1_round(float(inp)))
        assert got == float(exp), (inp, got, exp)
        assert not np.signbit(got) or got != 0.0


def test_e2m1_round_is_nearest_grid_point():
    rng = np.random.default_rng(71)
    v = rng.uniform(-7.5, 7.5, 20000)
    r = MX.e2m1_round(v)
    grid = np.concatenate([-MX.E2M1_VALUES[::-1], MX.E2M1_VALUES])
    dist = np.abs(v[:, None] - grid[None, :]).min(axis=1)
    inside = np.abs(v) <= 6
    np.testing.assert_allclose(np.abs(v - r)[inside], dist[inside], rtol=0, atol=0)
    assert np.all(np.abs(r[~inside]) == 6)


def test_mx_block_golden():
    rows = _rows("mx_block.txt")
    e_exp = int(rows[0][0])
    vals = np.array([float(t) for t in rows[1][0].split()])
    want = np.array([float(t) for t in rows[1][1].split()])
    q, e = MX.mx_quantize(vals[None, :], axis=1)
    assert int(e[0, 0]) == e_exp
    np.testing.assert_array_equal(q[0], want)


def test_mx_scale_properties():
    rng = np.random.default_rng(72)
    v = rng.standard_normal((40, 256)) * np.exp(rng.uniform(-20, 20, (40, 1)))
    v[3, 64:96] = 0.0
    q, e = MX.mx_quantize(v, axis=1)
    amax = np.abs(v.reshape(40, 8, 32)).max(-1)
    nz = amax > 0
    r = amax * np.ldexp(1.0, -e)
    assert np.all((r[nz] >= 4) & (r[nz] < 8))
    assert e[3, 2] == -127 and np.all(q[3, 64:96] == 0)
    assert set(np.unique(np.abs(q))) <= set(MX.E2M1_VALUES)
    # the block maximum maps to 4 or 6 (4 <= amax / 2^e < 8, then RNE + saturation)
    qa = np.abs(q.reshape(40, 8, 32)).max(-1)
    assert np.all(np.isin(qa[nz], [4.0, 6.0]))


def test_mx_product_bruteforce():
    rng = np.random.default_rng(73)
    M, K, N = 3, 96, 4
    qx = MX.e2m1_decode(rng.integers(0, 16, (M, K)))
    qw = MX.e2m1_decode(rng.integers(0, 16, (K, N)))
    ex = rng.integers(-10, 10, (M, K // 32))
    ew = rng.integers(-10, 10, (K // 32, N))
    np.testing.assert_array_equal(MX.mx_product(qx, ex, qw, ew), MX.mx_product_bruteforce(qx, ex, qw, ew))


def test_forward_mx_matches_dequantized_definition():
    wl = workloads.custom_workload(48, 256, 80, seed=74, n_out=3, bias=True)
    Lr = wl.layers[0]
    p = MX.prepare_mx(Lr.weight, wl.act_absmax(), rank=16)
    Y, parts = MX.forward_mx(wl.x, p, bias=Lr.bias, out="f64", return_parts=True)
    deq_x = parts["qx"] * np.repeat(np.ldexp(1.0, parts["ex"]), 32, axis=1)
    deq_w = p["qw"] * np.repeat(np.ldexp(1.0, p["ew"]), 32, axis=0)
    la = (O.bf16(parts["x_hat"]) @ p["L1"]).astype(np.float32).astype(np.float64)
    ref = deq_x @ deq_w + O.bf16(la) @ p["L2"] + Lr.bias[None, :]
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12)


def test_mx_residual_and_activation_reconstruct():
    """Dequantized MXFP4 residual is within half an E2M1 step (times the block
    scale) of R wherever no saturation happens."""
    wl = workloads.custom_workload(16, 256, 64, seed=75, n_out=3)
    p = MX.prepare_mx(wl.layers[0].weight, wl.act_absmax(), rank=32)
    s = np.repeat(np.ldexp(1.0, p["ew"]), 32, axis=0)
    err = np.abs(p["R"] - p["qw"] * s)
    half_step = np.where(np.abs(p["qw"]) < 2, 0.25, np.where(np.abs(p["qw"]) < 4, 0.5, 1.0)) * s
    sat = np.abs(p["R"]) / s > 6
    assert np.all(err[~sat] <= half_step[~sat])


def test_mx_error_story():
    """MXFP4: rank 32 beats rank 0 against fp64 X W; both far below 1."""
    wl = workloads.make_workload("tiny")
    x, w = wl.x, wl.layers[0].weight
    ref = O.reference_fp64(x, w)
    a = wl.act_absmax()
    e0 = O.rel_fro(MX.forward_mx(x, MX.prepare_mx(w, a, rank=0)), ref)
    e32 = O.rel_fro(MX.forward_mx(x, MX.prepare_mx(w, a, rank=32)), ref)
    assert e32 < e0 < 0.5


def test_prepared_bytes_mx_closed_form():
    """Bytes counted from the prepared arrays (codes packed two per byte, one
    E8M0 byte per block, bf16 factors, fp32 smooth_inv)."""
    wl = workloads.custom_workload(16, 256, 128, seed=76)
    p = MX.prepare_mx(wl.layers[0].weight, wl.act_absmax(), rank=32)
    codes = MX.e2m1_encode(p["qw"].T)
    nbytes = (O.pack_int4(codes).nbytes + p["ew"].astype(np.uint8).nbytes
              + 2 * (p["L1"].size + p["L2"].size) + p["smooth_inv"].astype(np.float32).nbytes)
    assert nbytes == MX.prepared_bytes_mx(256, 128, 32)
    # FLUX MLP-up layer: the same ~3.6x reduction from bf16 as the INT4 layer
    ratio = 2 * 3072 * 12288 / MX.prepared_bytes_mx(3072, 12288, 32)
    assert 3.5 < ratio < 3.7


def test_mx_decision_band_hand_worked():
    """Block absmax exactly 4 = 2^2: exponent 2 - 2 = 0; a hair below, 1 - 2 =
    -1.  With exponent 0 the values round on the E2M1 grid 0, 0.5, 1, 1.5, 2,
    3, 4, 6 with ties to the even code: 2.5 -> 2, 0.25 -> 0, 3.5 -> 4,
    -1.25 -> -1, 1.75 -> 2; a band of 1e-6 around each tie admits both
    neighbours."""
    x = np.zeros((1, 32))
    x[0, :6] = [4.0, 2.5, 0.25, 3.5, -1.25, 1.75]
    e_lo, e_hi, q_lo, q_hi = MX.activation_decision_band_mx(x, 0.0)
    assert e_lo[0, 0] == e_hi[0, 0] == 0
    assert list(q_lo[0, :6]) == list(q_hi[0, :6]) == [4.0, 2.0, 0.0, 4.0, -1.0, 2.0]
    e_lo, e_hi, q_lo, q_hi = MX.activation_decision_band_mx(x, 1e-6, exponents=np.zeros((1, 1)))
    assert (e_lo[0, 0], e_hi[0, 0]) == (-1, 0)
    assert list(q_lo[0, :6]) == [4.0, 2.0, 0.0, 3.0, -1.5, 1.5]
    assert list(q_hi[0, :6]) == [4.0, 3.0, 0.5, 4.0, -1.0, 2.0]


def test_mx_decision_band_zero_width_is_the_quantizer():
    rng = np.random.default_rng(6)
    x = O.bf16(rng.standard_normal((40, 256)) * np.where(rng.random(256) < 0.05, 30.0, 1.0))
    si = O.fp32(1.0 / (0.5 + rng.random(256)))
    q, e, xh = MX.quantize_activation_mx(x, si, act="gelu_tanh")
    e_lo, e_hi, q_lo, q_hi = MX.activation_decision_band_mx(xh, 0.0)
    np.testing.assert_array_equal(e_lo, e)
    np.testing.assert_array_equal(e_hi, e)
    np.testing.assert_array_equal(q_lo, q)
    np.testing.assert_array_equal(q_hi, q)
