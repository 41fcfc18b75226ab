"""Pins for the CPU oracle: each test checks it against something other than
itself (library routines, closed forms, brute force, hand-worked fixtures)."""
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([p.strip() for p in line.split("|")])
    return rows


# ---------------------------------------------------------------- rounding
def test_fp32_rounding_matches_numpy():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
                        [1 + 2 ** -24, 1 + 3 * 2 ** -24, 2 ** -149 * 1.5, 2 ** -149 * 2.5, 3.5e38, -0.0]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(O.fp32(x), ref)


def test_fp16_rounding_matches_numpy():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
                        [65504.0, 65519.99, 65520.0, 2 ** -24 * 0.5, 2 ** -24 * 1.5, 2 ** -25 * 1.0001,
                         1 + 2 ** -11, 1 + 3 * 2 ** -11]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(O.fp16(x), ref)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    x32 = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    # exact ties: 1 + 2^-8 and 1 + 3*2^-8 (bf16 has 7 stored fraction bits)
    x32 = np.concatenate([x32, np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], np.float32)])
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16(x32.astype(np.float64)), ref)


# ---------------------------------------------------------------- smoothing
def test_smoothing_closed_form():
    # weight [N=3][K=4]; per-input-channel maxima over outputs: 1, 0.25, 2, 0.5
    w = np.array([[1.0, -0.25, 0.5, 0.5],
                  [-0.5, 0.125, -2.0, 0.25],
                  [0.25, 0.0625, 1.0, -0.5]])
    a = np.array([4.0, 9.0, 2.0, 0.0], np.float32)
    si, lam = O.smoothing_factors(a, w)
    # lambda = sqrt(a / w): 2, 6, 1, sqrt(1e-5 / 0.5) (eps floor on a)
    expect = np.array([2.0, 6.0, 1.0, np.sqrt(1e-5 / 0.5)])
    np.testing.assert_array_equal(si, np.float32(1.0 / expect).astype(np.float64))
    np.testing.assert_allclose(lam * si, 1.0, rtol=2 ** -52)
    # the smoothed weight has the factor on input channels (rows of W = weight^T)
    W_hat = O.smooth_weight(w, lam)
    np.testing.assert_allclose(W_hat, (lam[:, None] * w.T), rtol=0)


def test_smoothing_alpha_golden():
    # alpha != 0.5 takes the general power form; hand-worked closed forms
    for al, a, w, inv in _read_golden("smoothing_alpha.txt"):
        si, lam = O.smoothing_factors(np.array([float(a)], np.float32),
                                      np.array([[float(w)]]), alpha=float(al))
        assert si[0] == float(np.float32(float(inv))), (al, a, w, si[0], inv)
        assert lam[0] * si[0] == pytest.approx(1.0, rel=2 ** -52)
    # alpha = 0.5 through the general form agrees with the square root form
    rng = np.random.default_rng(9)
    a = np.float32(rng.uniform(0.01, 50, 64))
    w = rng.standard_normal((8, 64))
    s_sqrt, _ = O.smoothing_factors(a, w, alpha=0.5)
    s_pow, _ = O.smoothing_factors(a, w, alpha=0.5 + 1e-15)
    np.testing.assert_allclose(s_pow, s_sqrt, rtol=1e-6)


# ---------------------------------------------------------------- invariants
def _pow2_lambda_case(M=24, K=128, N=40, seed=5):
    rng = np.random.default_rng(seed)
    x = O.bf16(rng.standard_normal((M, K)) * 3)
    w = O.bf16(rng.standard_normal((N, K)) * 0.02)
    e = rng.integers(-3, 4, K)
    wmax = np.abs(w).max(axis=0)
    a = (wmax * 4.0 ** e).astype(np.float32)     # exact: bf16 * power of 4
    return x, w, a, e


def test_rank0_quant_off_is_exact_matmul():
    """Rank 0, no quantization, power-of-two lambda: Y == X W bit for bit."""
    x, w, a, e = _pow2_lambda_case()
    p = O.prepare(w, a, rank=0)
    np.testing.assert_array_equal(p["lam"], 2.0 ** e)
    y = O.forward(x, p, out="f64", quantize=False)
    np.testing.assert_array_equal(y, O.reference_fp64(x, w))


@pytest.mark.parametrize("rank", [1, 8, 32])
def test_lambda_cancels_any_rank(rank):
    wl = workloads.custom_workload(64, 256, 96, seed=11, n_out=3)
    x, w = wl.x, wl.layers[0].weight
    p = O.prepare(w, wl.act_absmax(), rank=rank, round_factors=False)
    y = O.forward(x, p, out="f64", quantize=False)
    assert O.rel_fro(y, O.reference_fp64(x, w)) < 1e-13
    # the branch must be present: dropping it leaves a large error
    p2 = dict(p, L1=np.zeros_like(p["L1"]), L2=np.zeros_like(p["L2"]))
    assert O.rel_fro(O.forward(x, p2, out="f64", quantize=False), O.reference_fp64(x, w)) > 1e-2


def test_full_rank_leaves_zero_residual():
    wl = workloads.custom_workload(32, 128, 64, seed=12)
    p = O.prepare(wl.layers[0].weight, wl.act_absmax(), rank=64, round_factors=False)
    assert np.linalg.norm(p["R"]) <= 1e-12 * np.linalg.norm(p["W_hat"])


def test_eckart_young_against_eigh():
    """Residual of the top-r split equals sqrt(sum of the discarded
    eigenvalues of W_hat^T W_hat) and L1 L2 is the projection onto the top-r
    left eigenvectors of W_hat W_hat^T (independent LAPACK routine)."""
    wl = workloads.custom_workload(64, 192, 128, seed=13, n_out=6)
    r = 16
    p = O.prepare(wl.layers[0].weight, wl.act_absmax(), rank=r, round_factors=False)
    Wh = p["W_hat"]
    ev = np.sort(np.linalg.eigvalsh(Wh.T @ Wh))[::-1]
    res = np.linalg.norm(Wh - p["L1"] @ p["L2"])
    np.testing.assert_allclose(res, np.sqrt(ev[r:].sum()), rtol=1e-9)
    evl, U = np.linalg.eigh(Wh @ Wh.T)
    Ur = U[:, np.argsort(evl)[::-1][:r]]
    np.testing.assert_allclose(p["L1"] @ p["L2"], Ur @ (Ur.T @ Wh), atol=1e-10 * np.abs(Wh).max())


# ---------------------------------------------------------------- integer products
def test_group_products_bruteforce():
    rng = np.random.default_rng(21)
    M, K, N = 8, 128, 8
    qx = rng.integers(-8, 8, (M, K))
    qw = rng.integers(-8, 8, (K, N))
    qx[0, :64] = -8
    qw[:64, 0] = -8                                 # the extreme P = 4096
    P = O.w4a4_product_bruteforce(qx.tolist(), qw.tolist(), 64)
    assert P[0][0][0] == 4096
    ones_x = np.ones((M, 2))
    ones_w = np.ones((2, N))
    acc = O.w4a4_product(qx, ones_x, qw, ones_w, 64)
    np.testing.assert_array_equal(acc, np.array(P[0]) + np.array(P[1]))
    # non-uniform scales, each group weighted separately
    sx = O.fp16(rng.uniform(0.01, 1, (M, 2)))
    sw = O.fp16(rng.uniform(0.01, 1, (2, N)))
    acc = O.w4a4_product(qx, sx, qw, sw, 64)
    ref = sum(sx[:, g][:, None] * sw[g][None, :] * np.array(P[g], float) for g in range(2))
    np.testing.assert_allclose(acc, ref, rtol=1e-14)


def test_group_product_equals_dequantized_matmul():
    rng = np.random.default_rng(22)
    M, K, N, g = 16, 256, 24, 64
    qx = rng.integers(-8, 8, (M, K))
    qw = rng.integers(-8, 8, (K, N))
    sx = O.fp16(rng.uniform(0.01, 1, (M, K // g)))
    sw = O.fp16(rng.uniform(0.01, 1, (K // g, N)))
    deq_x = qx * np.repeat(sx, g, axis=1)
    deq_w = qw * np.repeat(sw, g, axis=0)
    np.testing.assert_allclose(O.w4a4_product(qx, sx, qw, sw, g), deq_x @ deq_w, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- quantizers
def test_activation_quant_golden():
    rows = _read_golden("act_quant_groups.txt")
    x = np.zeros((1, 64 * len(rows)))
    exp_s, exp_q = [], np.zeros(64 * len(rows), np.int64)
    for r in rows:
        g = int(r[0])
        vals = [float(v) for v in r[1].split()]
        x[0, 64 * g:64 * g + len(vals)] = vals
        exp_s.append(float(r[2]))
        codes = [int(v) for v in r[3].split()]
        exp_q[64 * g:64 * g + len(codes)] = codes
    q, s, _ = O.quantize_activation(x, np.ones(x.shape[1]), 64)
    np.testing.assert_array_equal(s[0], exp_s)
    np.testing.assert_array_equal(q[0], exp_q)


def test_weight_quant_golden():
    (r,) = _read_golden("weight_quant_group.txt")
    vals = [float(v) for v in r[0].split()]
    R = np.zeros((64, 1))
    R[:len(vals), 0] = vals
    q, s = O.quantize_weight_residual(R, 64)
    assert s[0, 0] == float(r[1])
    np.testing.assert_array_equal(q[:len(vals), 0], [int(v) for v in r[2].split()])
    assert np.all(q[len(vals):, 0] == 0)


def test_activation_quant_matches_float32_arithmetic():
    """The fp64-emulated fp32 rounding points agree with numpy float32
    arithmetic (IEEE single operations) on random smoothed data."""
    wl = workloads.custom_workload(64, 512, 64, seed=23, n_out=5)
    si, _ = O.smoothing_factors(wl.act_absmax(), wl.layers[0].weight)
    q, s, xh = O.quantize_activation(wl.x, si, 64)
    x32 = wl.x.astype(np.float32)
    xh32 = x32 * si.astype(np.float32)[None, :]
    a = np.abs(xh32.reshape(64, -1, 64)).max(-1)
    s32 = a / np.float32(7.0)
    s16 = s32.astype(np.float16).astype(np.float32)
    rcp = np.where(s16 == 0, np.float32(0), np.float32(1.0) / np.where(s16 == 0, np.float32(1), s16))
    q32 = np.clip(np.rint(xh32.reshape(64, -1, 64) * rcp[..., None]), -8, 7).reshape(64, -1)
    np.testing.assert_array_equal(xh, xh32.astype(np.float64))
    np.testing.assert_array_equal(s, s16.astype(np.float64))
    np.testing.assert_array_equal(q, q32.astype(np.int64))


def test_quantizer_properties():
    rng = np.random.default_rng(24)
    x = O.bf16(rng.standard_normal((32, 256)) * rng.uniform(0.1, 50, (32, 1)))
    x[3, 64:128] = 0.0
    q, s, xh = O.quantize_activation(x, np.ones(256), 64)
    assert q.min() >= -7 and q.max() <= 7          # absmax/7 never yields -8
    assert s[3, 1] == 0 and np.all(q[3, 64:128] == 0)
    xg, qg = xh.reshape(32, 4, 64), q.reshape(32, 4, 64)
    idx = np.abs(xg).argmax(-1)
    top = np.take_along_axis(qg, idx[..., None], -1)[..., 0]
    assert np.all((np.abs(top) == 7) | (s == 0))
    err = np.abs(xg - qg * s[..., None])
    assert np.all(err <= s[..., None] / 2 * (1 + 2 ** -9) + 1e-300)


def test_pack_golden_and_roundtrip():
    for r in _read_golden("pack_bytes.txt"):
        codes = np.array([[int(v) for v in r[0].split()]])
        expect = np.array([[int(v, 16) for v in r[1].split()]], np.uint8)
        np.testing.assert_array_equal(O.pack_int4(codes), expect)
    allc = np.arange(-8, 8)
    grid = np.stack(np.meshgrid(allc, allc), -1).reshape(1, -1)
    np.testing.assert_array_equal(O.unpack_int4(O.pack_int4(grid)), grid)


def test_gelu_matches_torch():
    x = np.linspace(-8, 8, 4001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    np.testing.assert_allclose(O.gelu_tanh(x), ref, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- end to end
def test_forward_matches_dequantized_definition():
    """The whole forward equals dequantize(Q4(X_hat)) dequantize(Q4(R)) +
    bf16(lora_act) L2 + bias, written with independent numpy pieces."""
    wl = workloads.custom_workload(48, 256, 80, seed=25, n_out=3, bias=True)
    L = wl.layers[0]
    p = O.prepare(L.weight, wl.act_absmax(), rank=16)
    Y, parts = O.forward(wl.x, p, bias=L.bias, out="f64", return_parts=True)
    deq_x = parts["qx"] * np.repeat(parts["sx"], 64, axis=1)
    deq_w = p["qw"] * np.repeat(p["sw"], 64, axis=0)
    la = (O.bf16(parts["x_hat"]) @ p["L1"]).astype(np.float32).astype(np.float64)
    la16 = torch.from_numpy(la.astype(np.float32)).to(torch.bfloat16).double().numpy()
    ref = deq_x @ deq_w + la16 @ p["L2"] + L.bias[None, :]
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12)


def test_error_story_low_rank_helps():
    """no smoothing r=0 > smoothing r=0 > smoothing r=32 (error vs fp64 X W)."""
    wl = workloads.make_workload("tiny")
    x, w = wl.x, wl.layers[0].weight
    ref = O.reference_fp64(x, w)
    a = wl.act_absmax()
    p_plain = O.prepare(w, np.abs(w).max(axis=0).astype(np.float32), rank=0)  # lambda = 1
    assert np.all(p_plain["lam"] == 1.0)
    e_plain = O.rel_fro(O.forward(x, p_plain), ref)
    e_r0 = O.rel_fro(O.forward(x, O.prepare(w, a, rank=0)), ref)
    e_r32 = O.rel_fro(O.forward(x, O.prepare(w, a, rank=32)), ref)
    assert e_plain > e_r0 > e_r32
    assert e_r32 < 0.1


def test_prepared_bytes_closed_form():
    wl = workloads.custom_workload(16, 256, 128, seed=26)
    p = O.prepare(wl.layers[0].weight, wl.act_absmax(), rank=32)
    nbytes = (O.pack_int4(p["qw"].T).nbytes + p["sw"].astype(np.float16).nbytes
              + 2 * (p["L1"].size + p["L2"].size) + p["smooth_inv"].astype(np.float32).nbytes)
    assert nbytes == O.prepared_bytes(256, 128, 32)
    # FLUX MLP-up layer: ~3.6x smaller than bf16 (the card states about 4x)
    ratio = 2 * 3072 * 12288 / O.prepared_bytes(3072, 12288, 32)
    assert 3.5 < ratio < 3.7


# ---------------------------------------------------------------- unfused comparison path
def _hand_prep(K=64, N=8, rank=16):
    """smooth_inv = 1, weight codes and scales and factors set by hand."""
    qw = np.zeros((K, N))
    sw = np.ones((K // 64, N))
    L1 = np.zeros((K, rank))
    L2 = np.zeros((rank, N))
    return dict(group=64, smooth_inv=np.ones(K, np.float32), qw=qw, sw=sw, L1=L1, L2=L2)


def test_unfused_double_rounding_worked_example():
    """Worked by hand.  Row 0 of X is (7, 1, 0, ...): absmax 7, scale 1,
    codes (7, 1).  Weight column 0 has codes (7, 7) and scale 4, so the 4-bit
    product is 4 * (7*7 + 1*7) = 224; bias 33 makes 257.  L1[1, 0] = 1 and
    L2[0, 0] = 1 give a low-rank term of exactly 1.
    Fused: bf16(257 + 1) = 258 (representable: 8 significant bits).
    Unfused: bf16(257) = 256 (257 lies halfway between 256 and 258; ties go
    to the even significand, 256), then bf16(256 + 1) = 256 again."""
    p = _hand_prep()
    p["qw"][0, 0] = p["qw"][1, 0] = 7
    p["sw"][0, 0] = 4.0
    p["L1"][1, 0] = 1.0
    p["L2"][0, 0] = 1.0
    x = np.zeros((2, 64))
    x[0, 0], x[0, 1] = 7.0, 1.0
    bias = np.zeros(8)
    bias[0] = 33.0
    fused = O.forward(x, p, bias=bias)
    unfused = O.forward_unfused(x, p, bias=bias)
    assert fused[0, 0] == 258.0
    assert unfused[0, 0] == 256.0
    # every other output is an exactly representable small integer: no rounding anywhere
    mask = np.ones_like(fused, bool)
    mask[0, 0] = False
    np.testing.assert_array_equal(fused[mask], unfused[mask])
    assert unfused[1, 0] == 33.0 and unfused[0, 1] == 0.0


def _half_ulp_bf16(v):
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - 8)


def test_unfused_within_two_roundings_of_exact():
    """Random layer: the unfused path is the exact fused value rounded twice,
    so |unfused - exact| <= half an ulp of the intermediate plus half an ulp
    of the result; at rank 0 it coincides with the fused forward."""
    wl = workloads.custom_workload(64, 256, 96, seed=27, n_out=3, bias=True)
    L = wl.layers[0]
    p = O.prepare(L.weight, wl.act_absmax(), rank=32)
    exact, parts = O.forward(wl.x, p, bias=L.bias, out="f64", return_parts=True)
    y0 = parts["acc"] + L.bias[None, :]
    un = O.forward_unfused(wl.x, p, bias=L.bias)
    bound = _half_ulp_bf16(y0) + _half_ulp_bf16(un) * (1 + 1e-12)
    assert np.all(np.abs(un - exact) <= bound)
    assert np.any(un != O.forward(wl.x, p, bias=L.bias))  # the extra rounding shows
    p0 = O.prepare(L.weight, wl.act_absmax(), rank=0)
    np.testing.assert_array_equal(O.forward_unfused(wl.x, p0, bias=L.bias), O.forward(wl.x, p0, bias=L.bias))


# ---------------------------------------------------------------- fused QKV epilogue
def test_rms_norm_matches_torch_and_closed_form():
    rng = np.random.default_rng(28)
    v = rng.standard_normal((5, 3, 128)) * 3
    g = 1 + 0.1 * rng.standard_normal(128)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(v), (128,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(v, g, 1e-6), ref, rtol=1e-13, atol=1e-13)
    # hand-worked: a head of all 2s has rms 2 and normalizes to g (eps 0)
    np.testing.assert_allclose(O.rms_norm(np.full(128, 2.0), g, 0.0), g, rtol=1e-15)
    # scale invariance
    np.testing.assert_allclose(O.rms_norm(7 * v, g, 0.0), O.rms_norm(v, g, 0.0), rtol=1e-13)


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(29)
    M, H, D = 6, 2, 128
    v = rng.standard_normal((M, H, D))
    ang = rng.uniform(-np.pi, np.pi, (M, D // 2))
    out = O.rope(v, np.cos(ang), np.sin(ang))
    z = (v[..., 0::2] + 1j * v[..., 1::2]) * np.exp(1j * ang)[:, None, :]
    np.testing.assert_allclose(out[..., 0::2], z.real, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(out[..., 1::2], z.imag, rtol=1e-13, atol=1e-13)
    # quarter turn maps (a, b) to (-b, a); pair norms are preserved
    q = O.rope(v, np.zeros((M, D // 2)), np.ones((M, D // 2)))
    np.testing.assert_array_equal(q[..., 0::2], -v[..., 1::2])
    np.testing.assert_array_equal(q[..., 1::2], v[..., 0::2])
    np.testing.assert_allclose(np.hypot(out[..., 0::2], out[..., 1::2]), np.hypot(v[..., 0::2], v[..., 1::2]),
                               rtol=1e-13)


def test_forward_qkv_composition():
    """V columns are the plain projection bit for bit; with unit norm weights
    and zero angles, Q and K heads have unit RMS before rounding."""
    wl = workloads.custom_workload(40, 256, 768, seed=30, n_out=3, bias=True)
    L = wl.layers[0]
    p = O.prepare(L.weight, wl.act_absmax(), rank=16)
    ones = np.ones(128)
    cos = np.ones((40, 64))
    sin = np.zeros((40, 64))
    Y = O.forward_qkv(wl.x, p, L.bias, ones, ones, cos, sin, out="f64")
    plain = O.forward(wl.x, p, bias=L.bias, out="f64")
    np.testing.assert_array_equal(Y[:, 512:], plain[:, 512:])
    heads = Y[:, :512].reshape(40, 4, 128)
    np.testing.assert_allclose(np.sqrt(np.mean(heads ** 2, axis=-1)), 1.0, rtol=1e-5)  # eps = 1e-6
    # rotating then normalizing equals normalizing then rotating (rotation keeps the RMS)
    ang = np.random.default_rng(31).uniform(0, 6, (40, 64))
    Yr = O.forward_qkv(wl.x, p, L.bias, ones, ones, np.cos(ang), np.sin(ang), out="f64")
    np.testing.assert_allclose(np.sqrt(np.mean(Yr[:, :512].reshape(40, 4, 128) ** 2, axis=-1)), 1.0, rtol=1e-5)


# ---------------------------------------------------------------- MLP chain
def _chain_case(M=48, K=128, N=256, N2=192, seed=21, rank=16):
    wl = workloads.custom_workload(M, K, N, seed=seed, n_out=3, bias=True, second_N=N2)
    up, dn = wl.layers
    pu = O.prepare(up.weight, wl.act_absmax(), rank=rank)
    y_up = O.forward(wl.x, pu, bias=up.bias)
    a_dn = np.abs(O.gelu_tanh(y_up)).max(0).astype(np.float32)
    pd = O.prepare(dn.weight, a_dn, rank=rank)
    return wl, up, dn, pu, pd


def test_mlp_chain_one_slice_is_the_composition():
    wl, up, dn, pu, pd = _chain_case()
    ref = O.forward(O.forward(wl.x, pu, bias=up.bias), pd, act="gelu_tanh", bias=dn.bias)
    got = O.forward_mlp_chain(wl.x, pu, pd, up.bias, dn.bias, slice_cols=256)
    np.testing.assert_array_equal(got, ref)


def test_mlp_chain_slices_round_once_each():
    """With slices, lora_act differs from the whole-row down projection only
    by the fp32 rounding of the partials and of their running sum: at most
    one fp32 unit per slice and addition relative to the sum of magnitudes."""
    wl, up, dn, pu, pd = _chain_case(N=512)
    _, parts = O.forward_mlp_chain(wl.x, pu, pd, up.bias, dn.bias, slice_cols=128, return_parts=True)
    whole = O.lora_down(parts["x_hat"], pd["L1"])
    mag = O.bf16(np.abs(parts["x_hat"])) @ np.abs(pd["L1"])
    assert np.all(np.abs(parts["lora_act"] - whole) <= 2 * 4 * 2.0 ** -24 * mag + 1e-30)
    # and the codes are those of the composition's down layer
    q, s, _ = O.quantize_activation(O.forward(wl.x, pu, bias=up.bias), pd["smooth_inv"], 64, act="gelu_tanh")
    np.testing.assert_array_equal(parts["qx"], q)
    np.testing.assert_array_equal(parts["sx"], s)


def test_mlp_chain_rank0_and_partial_slice():
    # rank 0 skips the branch; a last slice narrower than slice_cols works
    wl, up, dn, pu, pd0 = _chain_case(rank=0, N=320)
    ref = O.forward(O.forward(wl.x, pu, bias=up.bias), pd0, act="gelu_tanh", bias=dn.bias)
    np.testing.assert_array_equal(O.forward_mlp_chain(wl.x, pu, pd0, up.bias, dn.bias, slice_cols=256), ref)
    wl, up, dn, pu, pd = _chain_case(N=320)
    y = O.forward_mlp_chain(wl.x, pu, pd, up.bias, dn.bias, slice_cols=256)
    ref = O.forward(O.forward(wl.x, pu, bias=up.bias), pd, act="gelu_tanh", bias=dn.bias)
    assert O.rel_fro(y, ref) < 1e-5


# ---------------------------------------------------------------- decision band
def test_decision_band_hand_worked():
    """Activation quantizer decisions under a relative input band, worked by
    hand.  Group absmax 7 (1 + 2^-11): a / 7 = 1 + 2^-11 is the midpoint of the
    fp16 values 1 and 1 + 2^-10, which rounds to even (1); a hair above, to
    1 + 2^-10.  With scale 1 the codes are rne of the values themselves:
    2.5 -> 2 and -2.5 -> -2 (ties to even), 6.5 -> 6, 0.5 -> 0, 2.4 -> 2; a
    band of 1e-6 around a tie admits both neighbours, around 2.4 only 2."""
    x = np.zeros((1, 64))
    x[0, :6] = [7.00341796875, 2.5, -2.5, 2.4, 6.5, 0.5]
    s_lo, s_hi, q_lo, q_hi = O.activation_decision_band(x, 0.0)
    assert s_lo[0, 0] == s_hi[0, 0] == 1.0
    assert list(q_lo[0, :6]) == list(q_hi[0, :6]) == [7, 2, -2, 2, 6, 0]
    s_lo, s_hi, q_lo, q_hi = O.activation_decision_band(x, 1e-6)
    assert (s_lo[0, 0], s_hi[0, 0]) == (1.0, 1.0 + 2.0 ** -10)
    assert list(q_lo[0, :6]) == [7, 2, -3, 2, 6, 0]
    assert list(q_hi[0, :6]) == [7, 3, -2, 2, 7, 1]
    assert not q_lo[0, 6:].any() and not q_hi[0, 6:].any()
    # with the upper scale every value shrinks by ~2^-10: no tie is left
    _, _, q_lo, q_hi = O.activation_decision_band(x, 1e-6, scales=s_hi)
    assert list(q_lo[0, :6]) == list(q_hi[0, :6]) == [7, 2, -2, 2, 6, 0]


def test_decision_band_zero_width_is_the_quantizer():
    """rel = 0 gives quantize_activation's scales and codes, element for element."""
    rng = np.random.default_rng(5)
    x = O.bf16(rng.standard_normal((48, 256)) * np.where(rng.random(256) < 0.05, 30.0, 1.0))
    si = O.fp32(1.0 / (0.5 + rng.random(256)))
    q, s, xh = O.quantize_activation(x, si, 64, act="gelu_tanh")
    s_lo, s_hi, q_lo, q_hi = O.activation_decision_band(xh, 0.0)
    np.testing.assert_array_equal(s_lo, s)
    np.testing.assert_array_equal(s_hi, s)
    np.testing.assert_array_equal(q_lo, q)
    np.testing.assert_array_equal(q_hi, q)
    # and a band that is wide enough to matter stays ordered and within one step
    s_lo, s_hi, q_lo, q_hi = O.activation_decision_band(xh, 1e-3, scales=s)
    assert np.all(s_lo <= s) and np.all(s <= s_hi)
    assert np.all(q_lo <= q) and np.all(q <= q_hi) and np.all(q_hi - q_lo <= 1)
