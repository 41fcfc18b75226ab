"""Pins for the AWQ W4A16 oracle: hand-worked group, error bound, brute
force, alpha = 0 reduces to plain round-to-nearest, the search's choice."""
import os

import numpy as np
import pytest

import oracle as O
import workloads
from oracle import awq_oracle as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append([p.strip() for p in line.split("|")])
    return out


def test_awq_group_golden():
    (s_exp, z_exp), (vals, codes) = _rows("awq_group.txt")
    w = np.zeros((1, 64))
    w[0, :4] = [float(t) for t in vals.split()]
    q, s, z = A.awq_quantize(w)
    assert s[0, 0] == float(s_exp) and z[0, 0] == int(z_exp)
    want = np.full(64, 5)
    want[:4] = [int(t) for t in codes.split()]
    np.testing.assert_array_equal(q[0], want)


def test_awq_dequant_error_bound():
    rng = np.random.default_rng(41)
    w = rng.standard_normal((32, 256)) * np.exp(rng.uniform(-5, 5, (32, 1)))
    q, s, z = A.awq_quantize(w)
    err = np.abs(w - A.awq_dequantize(q, s, z))
    srep = np.repeat(s, 64, axis=1)
    assert np.all(err <= srep * (1 + 1e-9))            # the zero point's rounding may clip by up to s/2
    assert np.mean(err <= srep / 2 + 1e-12) > 0.99
    assert q.min() >= 0 and q.max() <= 15


def test_awq_forward_matches_bruteforce():
    wl = workloads.awq_workload(3, K=128, N=8, Mc=16, seed=42)
    p = A.awq_prepare(wl["weight"], wl["x_cal"])
    y = A.awq_forward(wl["x"], p, out="f64")
    x_hat = O.bf16(O.fp32(wl["x"] * p["inv_scale"][None, :]))
    np.testing.assert_allclose(y, A.awq_forward_bruteforce(x_hat, p["q"], p["s"], p["z"]), rtol=1e-12, atol=1e-14)


def test_awq_alpha0_is_plain_rtn():
    wl = workloads.awq_workload(2, K=256, N=64, Mc=16, seed=43)
    p = A.awq_prepare(wl["weight"], wl["x_cal"], alpha=0.0)
    assert np.all(p["inv_scale"] == 1.0)
    q, s, z = A.awq_quantize(wl["weight"])
    np.testing.assert_array_equal(p["q"], q)
    np.testing.assert_array_equal(p["s"], s)


def test_awq_search_helps_on_outlier_channels():
    """The searched alpha is the argmin of the grid losses and beats plain
    round-to-nearest (alpha = 0) on inputs with outlier channels, also on
    fresh rows of the same distribution."""
    wl = workloads.awq_workload(64, K=512, N=256, Mc=32, seed=44)
    p = A.awq_prepare(wl["weight"], wl["x_cal"])
    assert p["alpha"] == A.ALPHA_GRID[int(np.argmin(p["losses"]))]
    assert p["alpha"] > 0 and min(p["losses"]) < p["losses"][0]
    ref = wl["x"] @ wl["weight"].T
    p0 = A.awq_prepare(wl["weight"], wl["x_cal"], alpha=0.0)
    e_search = O.rel_fro(A.awq_forward(wl["x"], p, out="f64"), ref)
    e_plain = O.rel_fro(A.awq_forward(wl["x"], p0, out="f64"), ref)
    assert e_search < e_plain


def test_awq_scale_cancels_without_quantization():
    """x_hat-free check of the scale bookkeeping: (x * inv) . (w * t) = x . w
    in fp64 because t is taken as 1 / inv."""
    wl = workloads.awq_workload(4, K=128, N=16, Mc=8, seed=45)
    p = A.awq_prepare(wl["weight"], wl["x_cal"], alpha=0.5)
    t = 1.0 / p["inv_scale"]
    lhs = (wl["x"] * p["inv_scale"][None, :]) @ (wl["weight"] * t[None, :]).T
    np.testing.assert_allclose(lhs, wl["x"] @ wl["weight"].T, rtol=1e-12, atol=1e-15)


def test_awq_channel_scale_golden():
    x = np.array([[1.0, -4.0, 0.0], [-2.0, 8.0, 0.0], [3.0, 0.0, 0.0]])
    for al, t in _rows("awq_channel_scale.txt"):
        got = A.awq_channel_scale(x, float(al))
        np.testing.assert_allclose(got, [float(v) for v in t.split()], rtol=1e-14)
    # two channels: t = 2^-alpha/2, 2^alpha/2 for mean |x| = 2, 4 and alpha = 0.5
    got = A.awq_channel_scale(x[:, :2], 0.5)
    np.testing.assert_allclose(got, [2 ** -0.25, 2 ** 0.25], rtol=1e-15)


def test_awq_search_loss_golden():
    w = np.zeros((1, 64))
    w[0, :16], w[0, 16:32], w[0, 32:] = 1.0, -1.0, 0.296875
    x = np.zeros((1, 64))
    x[0, :32], x[0, 32:] = 1.0, 16.0
    p = A.awq_prepare(w, x)
    for al, idx, err, loss in _rows("awq_search_loss.txt"):
        assert A.ALPHA_GRID[int(idx)] == float(al)
        assert p["losses"][int(idx)] == pytest.approx(float(loss), rel=1e-12)
        assert float(err) ** 2 == float(loss)
    # the chosen alpha does no worse than either worked alpha
    best = min(p["losses"])
    assert best <= 6.890625
    assert p["losses"][int(round(p["alpha"] * 20))] == best
    # the worked alpha = 0.5 codes of the group: B channels 15, A channels 14 / 0
    q = A.awq_prepare(w, x, alpha=0.5)
    assert q["z"][0, 0] == 7 and q["s"][0, 0] == 1195 / 16384
    np.testing.assert_array_equal(q["q"][0], [14] * 16 + [0] * 16 + [15] * 32)
