"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: INT4 codes, fp16 scales and int32 accumulators bit-exact; lora_act
within 1e-5 relative Frobenius (fp32 summation order); bf16 output within
1e-3 relative Frobenius of the oracle's bf16 output (the bar the layer's
specification sets; observed values are ~1e-6, i.e. rare 1-ulp flips).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from tests._helpers import (abi_to_oracle_prep, bf16_bits_to_f64, check_bf16_elementwise,
                            check_f32_elementwise, check_int4_codes_in_band, f64_to_bf16_bits, oracle_prep_to_abi)

S = pytest.importorskip("w4a4_rank_corrected_svdq_amd")
from w4a4_rank_corrected_svdq_amd import _lib as L  # noqa: E402

pytestmark = pytest.mark.gpu

Y_TOL = 1e-3
LORA_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert S.device_check(0) == 0, "device is not gfx950"
    torch.cuda.set_device(0)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_np_bf16(t):
    return bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))


def run_k1(x_bits, smooth_inv, lora_down_bits, rank, act=L.SVDQ_ACT_NONE):
    x = dev_bf16(x_bits)
    si = dev(np.asarray(smooth_inv, np.float32))
    ld = dev_bf16(lora_down_bits) if rank else None
    xc, xs, la = S.quant_act_lora_down(x, si, ld, rank, act=act)
    torch.cuda.synchronize()
    return xc, xs, la


def run_k2(xc, xs, abi, la, bias_bits, M, out_dtype=L.SVDQ_OUT_BF16):
    r = abi["rank"]
    y = S.gemm_w4a4_lora_up(xc, xs, dev(abi["w_codes"]), dev(abi["w_scales"]), la,
                            dev_bf16(abi["lora_up"]) if r else None,
                            dev_bf16(bias_bits) if bias_bits is not None else None,
                            M, abi["N"], abi["K"], r, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


def y_to_np(y):
    return y.double().cpu().numpy() if y.dtype == torch.float32 else to_np_bf16(y)


def check_y(y, yo, tol=Y_TOL):
    """Relative Frobenius error within ``tol`` and the elementwise bound of
    the output type (one bf16 ulp but for a 1e-4 fraction; fp32 within
    2^-14 (|y| + rms y))."""
    yg = y if isinstance(y, np.ndarray) else y_to_np(y)
    e = O.rel_fro(yg, yo)
    assert e < tol, e
    if isinstance(y, torch.Tensor) and y.dtype == torch.float32:
        check_f32_elementwise(yg, yo)
    else:
        check_bf16_elementwise(yg, yo)
    return e


def y_from_k1_outputs(xc, xs, la, po, bias=None, rows=None, out="bf16"):
    """The oracle's kernel-2 arithmetic on kernel 1's own outputs (codes,
    scales, lora_act): isolates kernel 2 where kernel 1 may legitimately
    differ from the oracle (tanh-GELU codes on a rounding boundary)."""
    rows = slice(None) if rows is None else rows
    qx = O.unpack_int4(xc.cpu().numpy()[rows])
    sx = xs.cpu().numpy().astype(np.float64).T[rows]
    y = O.w4a4_product(qx, sx, po["qw"], po["sw"], 64)
    if po["L1"].shape[1]:
        y = y + O.bf16(la.double().cpu().numpy()[rows]) @ po["L2"]
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return O.bf16(y) if out == "bf16" else O.fp32(y)


# ------------------------------------------------------------------ kernel 2: integer core
@pytest.mark.parametrize("M,N,K", [(300, 264, 256), (16, 128, 64), (129, 8, 128), (1, 136, 192),
                                   (200, 1032, 12288), (4000, 4104, 320)])
def test_int32_group_products_bit_exact(M, N, K):
    """Unit scales, rank 0, fp32 output: y = sum_k q_x q_w is an integer below
    2^24, so it is exact in fp32 whatever the order; compared bit for bit
    with the oracle's exact integer products (including -8 codes and the
    all -8 extreme P_g = 4096)."""
    rng = np.random.default_rng(M * 7 + N)
    qx = rng.integers(-8, 8, (M, K))
    qw = rng.integers(-8, 8, (K, N))
    qx[0, :64] = -8
    qw[:64, 0] = -8
    G = K // 64
    ones_x = np.ones((M, G))
    ones_w = np.ones((G, N))
    ref = O.w4a4_product(qx, ones_x, qw, ones_w, 64)
    assert ref[0, 0] == 4096 + (ref[0, 0] - 4096)  # integer-valued
    abi = dict(w_codes=O.pack_int4(qw.T), w_scales=np.ones((G, N), np.float16),
               lora_up=np.zeros((N, 0), np.uint16), rank=0, N=N, K=K)
    xc = dev(O.pack_int4(qx))
    xs = dev(np.ones((G, M), np.float16))
    y = run_k2(xc, xs, abi, None, None, M, out_dtype=L.SVDQ_OUT_F32)
    np.testing.assert_array_equal(y.double().cpu().numpy(), ref)


def test_int32_single_group_isolation():
    """Zero every group but one: the output equals that group's P_g alone."""
    M, N, K = 64, 128, 512
    rng = np.random.default_rng(5)
    for g in (0, 3, 7):
        qx = np.zeros((M, K), np.int64)
        qw = np.zeros((K, N), np.int64)
        qx[:, 64 * g:64 * g + 64] = rng.integers(-8, 8, (M, 64))
        qw[64 * g:64 * g + 64] = rng.integers(-8, 8, (64, N))
        G = K // 64
        abi = dict(w_codes=O.pack_int4(qw.T), w_scales=np.ones((G, N), np.float16),
                   lora_up=np.zeros((N, 0), np.uint16), rank=0, N=N, K=K)
        y = run_k2(dev(O.pack_int4(qx)), dev(np.ones((G, M), np.float16)), abi, None, None, M,
                   out_dtype=L.SVDQ_OUT_F32)
        np.testing.assert_array_equal(y.double().cpu().numpy(), qx @ qw)


# ------------------------------------------------------------------ kernel 1
def _small_case(M=300, K=512, N=264, rank=32, seed=41, bias=False, n_out=4):
    wl = workloads.custom_workload(M, K, N, seed=seed, n_out=n_out, bias=bias)
    Lr = wl.layers[0]
    po = O.prepare(Lr.weight, wl.act_absmax(), rank=rank)
    return wl, Lr, po, oracle_prep_to_abi(po)


# (4200, 256, 32) and (4111, 192, 64): more 16-row blocks than an MI355X has
# CUs, so kernel 1 runs its 32-row blocks
@pytest.mark.parametrize("M,K,rank", [(300, 512, 32), (1, 64, 16), (16, 128, 0), (257, 1024, 48),
                                      (64, 512, 128), (33, 256, 256), (4200, 256, 32), (4111, 192, 64),
                                      (8200, 128, 128)])
def test_k1_codes_scales_lora_act(M, K, rank):
    N = max(8, ((rank + 7) // 8) * 8, 64)
    wl, Lr, po, abi = _small_case(M, K, N, rank, seed=42 + M)
    x = wl.x.copy()
    x[M // 2] = 0.0                     # an all-zero token row
    xb = f64_to_bf16_bits(x)
    xc, xs, la = run_k1(xb, abi["smooth_inv"], abi["lora_down"], rank)
    q, s, xh = O.quantize_activation(x, po["smooth_inv"], 64)
    np.testing.assert_array_equal(xc.cpu().numpy(), O.pack_int4(q))
    np.testing.assert_array_equal(xs.cpu().numpy().astype(np.float64), s.T)
    if rank:
        ref = O.lora_down(xh, po["L1"])
        assert O.rel_fro(la.double().cpu().numpy(), ref) < LORA_TOL


@pytest.mark.parametrize("M,K", [(512, 1024), (4200, 256)])
def test_k1_gelu_codes_in_band(M, K):
    """tanh-GELU on load: the device GELU and the oracle's fp64 tanh differ by
    ~1e-6 relative, so a scale or code may differ only where the oracle's
    value lies that close to its rounding boundary: every scale and code
    equals the oracle's where its decision is unique and is one of the two
    candidates elsewhere.  M = 4200 has more 16-row blocks than an MI355X has
    CUs, so kernel 1 runs 32-row blocks of 8 waves, with the GELU prologue."""
    rank = 32
    wl, Lr, po, abi = _small_case(M, K, 64, rank, seed=43)
    xc, xs, la = run_k1(wl.x_bits, abi["smooth_inv"], abi["lora_down"], rank, act=L.SVDQ_ACT_GELU_TANH)
    q, s, xh = O.quantize_activation(wl.x, po["smooth_inv"], 64, act="gelu_tanh")
    qg = O.unpack_int4(xc.cpu().numpy())
    amb_s, amb_q = check_int4_codes_in_band(qg, xs.cpu().numpy().astype(np.float64).T, xh)
    assert amb_s <= 0.03 * s.size and amb_q <= 1e-4 * q.size   # the band is narrow
    assert O.rel_fro(la.double().cpu().numpy(), O.lora_down(xh, po["L1"])) < 1e-4


def test_k1_zero_and_tiny_inputs():
    M, K = 32, 256
    x = np.zeros((M, K))
    x[1, 3] = 2.0 ** -100                # far below the fp16 scale range: s = 0
    x[2, 70] = 1e-6
    si = np.ones(K, np.float32)
    xc, xs, _ = run_k1(f64_to_bf16_bits(O.bf16(x)), si, None, 0)
    q, s, _ = O.quantize_activation(O.bf16(x), si, 64)
    np.testing.assert_array_equal(xc.cpu().numpy(), O.pack_int4(q))
    np.testing.assert_array_equal(xs.cpu().numpy().astype(np.float64), s.T)


# ------------------------------------------------------------------ kernel 2 full epilogue
@pytest.mark.parametrize("rank,bias,out", [(0, False, "bf16"), (16, True, "bf16"), (32, False, "bf16"),
                                           (32, True, "f32"), (64, True, "bf16"), (128, False, "bf16"),
                                           (256, True, "bf16"), (48, False, "f32")])
def test_k2_output_parity(rank, bias, out):
    M, K, N = 300, 512, 264
    wl, Lr, po, abi = _small_case(M, K, N, rank, seed=44 + rank, bias=bias)
    Yo, parts = O.forward(wl.x, po, bias=Lr.bias, out=("f32" if out == "f32" else "bf16"), return_parts=True)
    xc = dev(O.pack_int4(parts["qx"]))
    xs = dev(parts["sx"].T.astype(np.float16))
    la = dev(parts["lora_act"].astype(np.float32)) if rank else None
    y = run_k2(xc, xs, abi, la, Lr.bias_bits if bias else None, M,
               out_dtype=L.SVDQ_OUT_F32 if out == "f32" else L.SVDQ_OUT_BF16)
    e = check_y(y, Yo)
    if out == "f32":
        assert e < 1e-5, e


# Kernel 2 has two tile forms: 256 x 256 (8 waves) when M is even and the
# grid has at least 192 such tiles, 128 x 128 otherwise.  These cases put the
# large form on ragged M and N edges (4000 = 15.6 tiles, 4104 = 16.03 tiles)
# with odd and single group counts and every epilogue option, and compare
# every output with the oracle.
LARGE_FORM = (4000, 4104)


@pytest.mark.parametrize("rank,bias,out,K", [(0, False, "bf16", 192), (32, True, "bf16", 192),
                                             (48, True, "f32", 192), (16, False, "bf16", 64),
                                             (32, False, "f32", 128), (256, True, "bf16", 320)])
def test_k2_large_form_parity(rank, bias, out, K):
    """K = 64 and 128 are one stage (the second group of K = 64 is past K);
    rank 256 runs the up projection in eight slices before the K loop."""
    M, N = LARGE_FORM
    wl, Lr, po, abi = _small_case(M, K, N, rank, seed=60 + rank, bias=bias)
    Yo, parts = O.forward(wl.x, po, bias=Lr.bias, out=("f32" if out == "f32" else "bf16"), return_parts=True)
    xc = dev(O.pack_int4(parts["qx"]))
    xs = dev(parts["sx"].T.astype(np.float16))
    la = dev(parts["lora_act"].astype(np.float32)) if rank else None
    od = L.SVDQ_OUT_F32 if out == "f32" else L.SVDQ_OUT_BF16
    y = run_k2(xc, xs, abi, la, Lr.bias_bits if bias else None, M, out_dtype=od)
    e = check_y(y, Yo)
    if out == "f32":
        assert e < 1e-5, e
    again = run_k2(xc, xs, abi, la, Lr.bias_bits if bias else None, M, out_dtype=od)
    assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32),
                       again.view(torch.int16) if again.dtype == torch.bfloat16 else again.view(torch.int32))


@pytest.mark.parametrize("shape", [(300, 512, 264), (128, 1024, 512), (5, 256, 1032)])
def test_end_to_end_parity(shape):
    M, K, N = shape
    wl, Lr, po, abi = _small_case(M, K, N, 32, seed=45 + M, bias=True)
    xc, xs, la = run_k1(wl.x_bits, abi["smooth_inv"], abi["lora_down"], 32)
    y = run_k2(xc, xs, abi, la, Lr.bias_bits, M)
    Yo = O.forward(wl.x, po, bias=Lr.bias)
    check_y(y, Yo)
    np.testing.assert_array_equal(xc.cpu().numpy(), O.pack_int4(O.quantize_activation(wl.x, po["smooth_inv"], 64)[0]))


def test_determinism_bitwise():
    M, K, N = 256, 512, 512
    wl, Lr, po, abi = _small_case(M, K, N, 32, seed=46)
    outs = []
    for _ in range(3):
        xc, xs, la = run_k1(wl.x_bits, abi["smooth_inv"], abi["lora_down"], 32)
        outs.append((xc.cpu().numpy(), xs.cpu().numpy(), la.cpu().numpy(),
                     run_k2(xc, xs, abi, la, None, M).view(torch.int16).cpu().numpy()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            np.testing.assert_array_equal(a, b)


def test_mlp_chain_gelu_small():
    """Up projection -> tanh-GELU fused into the down layer's kernel 1 ->
    down projection, GPU chain vs oracle chain (each side feeds its own
    intermediate; a rare 1-ulp bf16 difference in the intermediate can move
    a code, so the bar is on the final output)."""
    M, K, N = 256, 512, 2048
    wl = workloads.custom_workload(M, K, N, seed=47, n_out=4, second_N=512)
    up, down = wl.layers
    pu = O.prepare(up.weight, wl.act_absmax(), rank=32)
    y_up_o = O.forward(wl.x, pu)
    a_dn = np.abs(O.gelu_tanh(O.reference_fp64(wl.x, up.weight))).max(0).astype(np.float32)
    pd = O.prepare(down.weight, a_dn, rank=32)
    y_dn_o = O.forward(y_up_o, pd, act="gelu_tanh")
    au, ad = oracle_prep_to_abi(pu), oracle_prep_to_abi(pd)
    xc, xs, la = run_k1(wl.x_bits, au["smooth_inv"], au["lora_down"], 32)
    y_up = run_k2(xc, xs, au, la, None, M)
    check_y(y_up, y_up_o)
    x2 = S.quant_act_lora_down(y_up, dev(ad["smooth_inv"]), dev_bf16(ad["lora_down"]), 32,
                               act=L.SVDQ_ACT_GELU_TANH)
    y_dn = run_k2(*x2[:2], ad, x2[2], None, M)
    assert O.rel_fro(y_to_np(y_dn), y_dn_o) < Y_TOL
    # elementwise: the down layer's kernel 2 on its own kernel 1's outputs
    check_bf16_elementwise(y_to_np(y_dn), y_from_k1_outputs(*x2, pd))


# ------------------------------------------------------------------ unfused comparison path
def run_unfused(x_bits, abi, bias_bits, M, act=L.SVDQ_ACT_NONE):
    """Kernel 1 and kernel 2 at rank 0, then the separate down projection
    (re-reading x) and the separate up projection (read-modify-write of y)."""
    r, N, K = abi["rank"], abi["N"], abi["K"]
    x = dev_bf16(x_bits)
    si = dev(abi["smooth_inv"])
    xc, xs, _ = S.quant_act_lora_down(x, si, None, 0, act=act)
    y = S.gemm_w4a4_lora_up(xc, xs, dev(abi["w_codes"]), dev(abi["w_scales"]), None, None,
                            dev_bf16(bias_bits) if bias_bits is not None else None, M, N, K, 0)
    la = S.lora_down(x, si, dev_bf16(abi["lora_down"]), r, act=act)
    S.lora_up_add(la, dev_bf16(abi["lora_up"]), y)
    torch.cuda.synchronize()
    return xc, xs, la, y


@pytest.mark.parametrize("M,K,N,rank,bias", [(300, 512, 264, 32, True), (1, 64, 24, 16, False),
                                             (129, 1024, 520, 64, True), (64, 256, 136, 128, False),
                                             (33, 512, 256, 256, True)])
def test_unfused_branch_parity(M, K, N, rank, bias):
    """The unfused path against the oracle's unfused forward; its down
    projection is bit-identical to the fused kernel 1's (same kernel, no
    quantizer), and its 4-bit codes and scales to the fused ones."""
    wl, Lr, po, abi = _small_case(M, K, N, rank, seed=49 + M, bias=bias)
    bb = Lr.bias_bits if bias else None
    xc, xs, la, y = run_unfused(wl.x_bits, abi, bb, M)
    xc1, xs1, la1 = run_k1(wl.x_bits, abi["smooth_inv"], abi["lora_down"], rank)
    np.testing.assert_array_equal(xc.cpu().numpy(), xc1.cpu().numpy())
    np.testing.assert_array_equal(xs.cpu().numpy(), xs1.cpu().numpy())
    np.testing.assert_array_equal(la.cpu().numpy(), la1.cpu().numpy())
    q, s, xh = O.quantize_activation(wl.x, po["smooth_inv"], 64)
    assert O.rel_fro(la.double().cpu().numpy(), O.lora_down(xh, po["L1"])) < LORA_TOL
    Yo = O.forward_unfused(wl.x, po, bias=Lr.bias if bias else None)
    check_y(to_np_bf16(y), Yo)


def test_lora_up_add_in_place_parity():
    """The standalone up projection on oracle inputs: y0 bf16 and lora_act
    taken from the oracle, result against bf16(y0 + bf16(lora_act) L2)."""
    M, K, N, r = 200, 256, 392, 48
    wl, Lr, po, abi = _small_case(M, K, N, r, seed=50, bias=True)
    rng = np.random.default_rng(51)
    y0 = O.bf16(rng.standard_normal((M, N)) * 4)
    la = O.fp32(rng.standard_normal((M, r)) * 3)
    y = dev_bf16(f64_to_bf16_bits(y0))
    S.lora_up_add(dev(la.astype(np.float32)), dev_bf16(abi["lora_up"]), y)
    torch.cuda.synchronize()
    ref = O.bf16(y0 + O.bf16(la) @ po["L2"])
    got = to_np_bf16(y)
    check_y(got, ref)
    # at most a 1-ulp flip where fp32 summation order meets a rounding boundary
    assert (got != ref).mean() < 0.01


def test_unfused_full_size_sampled_rows():
    """The unfused path at the FLUX MLP-up shape [4096 x 3072] -> 12288,
    rank 32, sampled rows against the oracle's unfused forward."""
    wl = workloads.make_workload("mlp_pair")
    Lr = wl.layers[0]
    M, K, N, r = wl.M, Lr.K, Lr.N, 32
    rng = np.random.default_rng(9)
    a = wl.act_absmax()
    si, lam = O.smoothing_factors(a, Lr.weight)
    l1, l2 = _synthetic_factors(K, N, r, rng, scale=float(np.abs(lam).mean() * 0.02))
    po = O.prepare(Lr.weight, a, rank=r, factors=(l1, l2))
    abi = oracle_prep_to_abi(po)
    xc, xs, la, y = run_unfused(wl.x_bits, abi, Lr.bias_bits, M)
    rows = _sample_rows(M, rng)
    Yo = O.forward_unfused(wl.x[rows], po, bias=Lr.bias)
    check_y(to_np_bf16(y[torch.from_numpy(rows).cuda()]), Yo)
    assert torch.isfinite(y.float()).all()


# ------------------------------------------------------------------ FLUX shapes, sampled rows
FULL = {
    "attn_out": dict(name="attn_out", rank=32),
    "joint_qkv": dict(name="joint_qkv", rank=32),
    "mlp_up": dict(name="mlp_pair", rank=32),
    "rank_sweep_r32": dict(name="rank_sweep", rank=32),
    "rank_sweep_r64": dict(name="rank_sweep", rank=64),
    "rank_sweep_r128": dict(name="rank_sweep", rank=128),
}


def _sample_rows(M, rng, n=48):
    rows = np.unique(np.concatenate([np.arange(8), rng.choice(M, n - 16, replace=False), np.arange(M - 8, M)]))
    return rows


def _synthetic_factors(K, N, r, rng, scale):
    l1 = O.bf16(rng.standard_normal((K, r)) * scale)
    l2 = O.bf16(rng.standard_normal((r, N)) / np.sqrt(N))
    return l1, l2


@pytest.mark.parametrize("case", list(FULL))
def test_full_size_sampled_rows(case):
    """Both kernels at the FLUX shape, in the launch configuration the
    benchmark times.  Codes and scales of every row against the oracle's
    quantizer; lora_act and the output on a sample of rows (first, last and
    random ones).  The factors are seeded synthetic bf16 matrices so that the
    oracle's preparation needs no full-size SVD (the split itself is pinned
    at small sizes)."""
    wl = workloads.make_workload(FULL[case]["name"])
    Lr = wl.layers[0]
    M, K, N = wl.M, Lr.K, Lr.N
    r = FULL[case]["rank"]
    rng = np.random.default_rng(7)
    a = wl.act_absmax()
    si, lam = O.smoothing_factors(a, Lr.weight)
    l1, l2 = _synthetic_factors(K, N, r, rng, scale=float(np.abs(lam).mean() * 0.02))
    po = O.prepare(Lr.weight, a, rank=r, factors=(l1, l2))
    abi = oracle_prep_to_abi(po)
    xc, xs, la = run_k1(wl.x_bits, abi["smooth_inv"], abi["lora_down"], r)
    y = run_k2(xc, xs, abi, la, Lr.bias_bits, M)
    q_all, s_all, _ = O.quantize_activation(wl.x, po["smooth_inv"], 64)
    np.testing.assert_array_equal(xc.cpu().numpy(), O.pack_int4(q_all))
    np.testing.assert_array_equal(xs.cpu().numpy().astype(np.float64), s_all.T)
    del q_all, s_all
    rows = _sample_rows(M, rng)
    xr = wl.x[rows]
    Yo, parts = O.forward(xr, po, bias=Lr.bias, return_parts=True)
    assert O.rel_fro(la.double().cpu().numpy()[rows], parts["lora_act"]) < LORA_TOL
    yr = to_np_bf16(y[torch.from_numpy(rows).cuda()])
    check_y(yr, Yo)
    assert torch.isfinite(y.float()).all()


def test_full_size_mlp_down_gelu_sampled_rows():
    """Down projection shape (K = 12288) with tanh-GELU fused on load; the
    input is a seeded [4096][12288] bf16 activation with the same recipe."""
    M, K, N, r = 4096, 12288, 3072, 32
    wl = workloads.custom_workload(M, K, N, seed=48, n_out=61, factor=(20.0, 50.0))
    Lr = wl.layers[0]
    a = np.abs(O.gelu_tanh(wl.x)).max(0).astype(np.float32)
    rng = np.random.default_rng(8)
    si, lam = O.smoothing_factors(a, Lr.weight)
    l1, l2 = _synthetic_factors(K, N, r, rng, scale=float(np.abs(lam).mean() * 0.02))
    po = O.prepare(Lr.weight, a, rank=r, factors=(l1, l2))
    abi = oracle_prep_to_abi(po)
    xc, xs, la = run_k1(wl.x_bits, abi["smooth_inv"], abi["lora_down"], r, act=L.SVDQ_ACT_GELU_TANH)
    y = run_k2(xc, xs, abi, la, None, M)
    _, _, xh_all = O.quantize_activation(wl.x, po["smooth_inv"], 64, act="gelu_tanh")
    check_int4_codes_in_band(O.unpack_int4(xc.cpu().numpy()), xs.cpu().numpy().astype(np.float64).T, xh_all)
    del xh_all
    rows = _sample_rows(M, rng, 32)
    Yo = O.forward(wl.x[rows], po, act="gelu_tanh")
    yr = to_np_bf16(y[torch.from_numpy(rows).cuda()])
    assert O.rel_fro(yr, Yo) < Y_TOL
    check_bf16_elementwise(yr, y_from_k1_outputs(xc, xs, la, po, rows=rows))


def test_error_story_product_path():
    """Library preparation + both kernels on the attention-output shape:
    error against fp64 X W on sampled rows falls from rank 0 to rank 32
    (the low-rank branch absorbs what 4 bits cannot carry)."""
    wl = workloads.make_workload("attn_out")
    Lr = wl.layers[0]
    rows = _sample_rows(wl.M, np.random.default_rng(9), 64)
    ref = O.reference_fp64(wl.x[rows], Lr.weight)
    errs = {}
    for r in (0, 32):
        lin = S.SVDQW4A4Linear(S.prepare_weights(Lr.weight_bits, wl.act_absmax(), rank=r), None, "cuda")
        y = lin(dev_bf16(wl.x_bits))
        torch.cuda.synchronize()
        errs[r] = O.rel_fro(to_np_bf16(y[torch.from_numpy(rows).cuda()]), ref)
    assert errs[32] < errs[0] < 0.2, errs


def test_linear_module_with_oracle_prepared_arrays():
    """SVDQW4A4Linear built from the oracle's (possibly non-contiguous)
    arrays: the binding lays them out row-major before handing them over."""
    M, K, N = 256, 512, 520
    wl, Lr, po, abi = _small_case(M, K, N, 32, seed=49, bias=True)
    prep = dict(smooth_inv=po["smooth_inv"].astype(np.float32), w_codes=O.pack_int4(po["qw"].T),
                w_scales=po["sw"].astype(np.float16), lora_down=abi["lora_down"], lora_up=abi["lora_up"],
                rank=32, group=64, K=K, N=N)
    bias = torch.from_numpy(Lr.bias_bits.view(np.int16).copy()).view(torch.bfloat16)
    lin = S.SVDQW4A4Linear(prep, bias, "cuda:0")
    y = lin(dev_bf16(wl.x_bits))
    torch.cuda.synchronize()
    check_y(to_np_bf16(y), O.forward(wl.x, po, bias=Lr.bias))


@pytest.mark.parametrize("engine", ["fp6", "int8"])
def test_library_prepared_layer_against_oracle(engine):
    """Library preparation (smoothing, SVD split, INT4 residual) feeding both
    kernels of either engine, against the oracle's forward on the very
    arrays the library prepared, at three ranks and with bias."""
    for M, K, N, r in ((300, 512, 264, 32), (64, 1024, 520, 0), (129, 256, 392, 64)):
        wl = workloads.custom_workload(M, K, N, seed=64 + r, n_out=4, bias=True)
        Lr = wl.layers[0]
        p = S.prepare_weights(Lr.weight_bits, wl.act_absmax(), rank=r)
        po = abi_to_oracle_prep(p)
        lin = S.SVDQW4A4Linear(p, torch.from_numpy(Lr.bias_bits.view(np.int16).copy()).view(torch.bfloat16), "cuda",
                               engine=engine)
        assert lin.engine == engine
        y = lin(dev_bf16(wl.x_bits))
        torch.cuda.synchronize()
        check_y(to_np_bf16(y), O.forward(wl.x, po, bias=Lr.bias))


def test_checkpoint_round_trip_forward(tmp_path):
    """A layer saved to a checkpoint and loaded back computes bit-identical
    outputs, and matches the oracle on the prepared arrays it holds."""
    from w4a4_rank_corrected_svdq_amd import checkpoint as C
    M, K, N = 64, 512, 264
    wl = workloads.custom_workload(M, K, N, seed=62, n_out=4, bias=True)
    Lr = wl.layers[0]
    p = S.prepare_weights(Lr.weight_bits, wl.act_absmax(), rank=32)
    path = str(tmp_path / "ckpt.safetensors")
    C.save_prepared(path, {"proj": p}, {"proj": Lr.bias_bits})
    lin0 = S.SVDQW4A4Linear(p, torch.from_numpy(Lr.bias_bits.view(np.int16).copy()).view(torch.bfloat16), "cuda")
    lin1 = C.load_linears(path)["proj"]
    x = dev_bf16(wl.x_bits)
    y0, y1 = lin0(x), lin1(x)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y0.view(torch.int16).cpu().numpy(), y1.view(torch.int16).cpu().numpy())
    _, loaded = C.load_prepared(path)
    check_y(to_np_bf16(y1), O.forward(wl.x, abi_to_oracle_prep(loaded["proj"][0]), bias=Lr.bias))


def test_checkpoint_round_trip_mxfp4_and_awq(tmp_path):
    """MXFP4 and AWQ layers saved to one checkpoint and loaded back compute
    bit-identical outputs to the layers they were saved from."""
    from w4a4_rank_corrected_svdq_amd import checkpoint as C
    wl = workloads.custom_workload(64, 512, 264, seed=65, n_out=4, bias=True)
    Lr = wl.layers[0]
    pm = S.prepare_weights_mxfp4(Lr.weight_bits, wl.act_absmax(), rank=32)
    aw = workloads.awq_workload(3, K=512, N=256, Mc=8, seed=66)
    pa = S.awq_prepare(aw["weight_bits"], aw["x_cal_bits"])
    path = str(tmp_path / "ckpt.safetensors")
    C.save_prepared(path, {"proj": pm}, {"proj": Lr.bias_bits, "mod": aw["bias_bits"]}, awq_layers={"mod": pa})
    got = C.load_linears(path)
    bf = lambda b: torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16)  # noqa: E731
    ref_m = S.SVDQW4A4Linear(pm, bf(Lr.bias_bits), "cuda")
    ref_a = S.AWQW4A16Linear(pa, bf(aw["bias_bits"]), "cuda")
    assert isinstance(got["mod"], S.AWQW4A16Linear) and got["proj"].precision == "mxfp4"
    x = dev_bf16(wl.x_bits)
    xa = dev_bf16(aw["x_bits"])
    pairs = ((ref_m(x), got["proj"](x)), (ref_a(xa), got["mod"](xa)))
    torch.cuda.synchronize()
    for a, b in pairs:
        np.testing.assert_array_equal(a.view(torch.int16).cpu().numpy(), b.view(torch.int16).cpu().numpy())


# ------------------------------------------------------------------ fused QKV epilogue
def _qkv_inputs(M, seed, rope=True):
    (qb, qv), (kb, kv) = workloads.norm_weights(seed=seed)
    if rope:
        ang = np.random.default_rng(seed).uniform(-np.pi, np.pi, (M, 64))
        cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    else:
        cos = sin = None
    return qb, qv, kb, kv, cos, sin


def run_qkv(xc, xs, abi, la, bias_bits, M, qb, kb, cos, sin, out_dtype=L.SVDQ_OUT_BF16):
    r = abi["rank"]
    y = S.gemm_w4a4_lora_up_qkv(xc, xs, dev(abi["w_codes"]), dev(abi["w_scales"]), la,
                                dev_bf16(abi["lora_up"]) if r else None,
                                dev_bf16(bias_bits) if bias_bits is not None else None,
                                dev_bf16(qb), dev_bf16(kb),
                                dev(cos) if cos is not None else None, dev(sin) if sin is not None else None,
                                M, abi["N"], abi["K"], r, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M,heads,rank,bias,rope,out", [(300, 2, 32, True, True, "bf16"),
                                                        (300, 2, 32, True, True, "f32"),
                                                        (64, 1, 0, False, False, "bf16"),
                                                        (129, 3, 16, True, False, "f32")])
def test_qkv_epilogue_parity(M, heads, rank, bias, rope, out):
    """Projection + per-head Q/K RMSNorm + rotary embedding against the
    oracle's fused QKV operator; V columns bit-identical to the plain kernel."""
    K, N = 512, 3 * heads * 128
    wl, Lr, po, abi = _small_case(M, K, N, rank, seed=52 + M, bias=bias)
    qb, qv, kb, kv, cos, sin = _qkv_inputs(M, 53 + M, rope)
    Yo, parts = O.forward(wl.x, po, bias=Lr.bias, out="f64", return_parts=True)
    ref = O.forward_qkv(wl.x, po, Lr.bias, qv, kv, cos, sin, out=out)
    xc = dev(O.pack_int4(parts["qx"]))
    xs = dev(parts["sx"].T.astype(np.float16))
    la = dev(parts["lora_act"].astype(np.float32)) if rank else None
    od = L.SVDQ_OUT_F32 if out == "f32" else L.SVDQ_OUT_BF16
    y = run_qkv(xc, xs, abi, la, Lr.bias_bits if bias else None, M, qb, kb, cos, sin, out_dtype=od)
    check_y(y, ref, tol=(1e-5 if out == "f32" else Y_TOL))
    plain = run_k2(xc, xs, abi, la, Lr.bias_bits if bias else None, M, out_dtype=od)
    v0 = 2 * heads * 128
    np.testing.assert_array_equal(y[:, v0:].float().cpu().numpy(), plain[:, v0:].float().cpu().numpy())


@pytest.mark.parametrize("M,heads,out", [(4096, 11, "bf16"), (4096, 11, "f32"), (4000, 8, "bf16")])
def test_qkv_large_form_parity(M, heads, out):
    """The fused QKV epilogue on the 256 x 256 form: 11 heads (N = 4224, so
    one block holds the last Q head and the first K head, and the last block
    column is half full), or 8 heads on M = 4000 (the last block row holds
    160 rows, whose missing rotary rows are read as zeros and never stored);
    rank 16, bias, rotary tables; every output against the oracle, V columns
    bit-identical to the plain kernel."""
    K, rank = 256, 16
    N = 3 * heads * 128
    wl, Lr, po, abi = _small_case(M, K, N, rank, seed=62, bias=True)
    qb, qv, kb, kv, cos, sin = _qkv_inputs(M, 63, True)
    Yo, parts = O.forward(wl.x, po, bias=Lr.bias, out="f64", return_parts=True)
    ref = O.forward_qkv(wl.x, po, Lr.bias, qv, kv, cos, sin, out=out)
    xc = dev(O.pack_int4(parts["qx"]))
    xs = dev(parts["sx"].T.astype(np.float16))
    la = dev(parts["lora_act"].astype(np.float32))
    od = L.SVDQ_OUT_F32 if out == "f32" else L.SVDQ_OUT_BF16
    y = run_qkv(xc, xs, abi, la, Lr.bias_bits, M, qb, kb, cos, sin, out_dtype=od)
    check_y(y, ref, tol=(1e-5 if out == "f32" else Y_TOL))
    plain = run_k2(xc, xs, abi, la, Lr.bias_bits, M, out_dtype=od)
    v0 = 2 * heads * 128
    np.testing.assert_array_equal(y[:, v0:].float().cpu().numpy(), plain[:, v0:].float().cpu().numpy())


def test_qkv_full_size_sampled_rows():
    """The joint-stream QKV shape (4096 image + 512 text rows, 3072 -> 9216,
    rank 32, bias) with FLUX-style rotary tables, both kernels in the launch
    configuration the benchmark times, sampled rows against the oracle."""
    wl = workloads.make_workload("joint_qkv")
    Lr = wl.layers[0]
    M, K, N, r = wl.M, Lr.K, Lr.N, 32
    rng = np.random.default_rng(11)
    a = wl.act_absmax()
    si, lam = O.smoothing_factors(a, Lr.weight)
    l1, l2 = _synthetic_factors(K, N, r, rng, scale=float(np.abs(lam).mean() * 0.02))
    po = O.prepare(Lr.weight, a, rank=r, factors=(l1, l2))
    abi = oracle_prep_to_abi(po)
    (qb, qv), (kb, kv) = workloads.norm_weights(seed=12)
    cos, sin = workloads.rope_tables(512, 64)
    xc, xs, la = run_k1(wl.x_bits, abi["smooth_inv"], abi["lora_down"], r)
    y = run_qkv(xc, xs, abi, la, Lr.bias_bits, M, qb, kb, cos, sin)
    rows = _sample_rows(M, rng)
    ref = O.forward_qkv(wl.x[rows], po, Lr.bias, qv, kv, cos[rows], sin[rows])
    check_y(to_np_bf16(y[torch.from_numpy(rows).cuda()]), ref)
    assert torch.isfinite(y.float()).all()


@pytest.mark.parametrize("kind", [L.SVDQ_PROBE_MFMA_I8, L.SVDQ_PROBE_MFMA_FP4, L.SVDQ_PROBE_MFMA_FP6,
                                  L.SVDQ_PROBE_DEQUANT, L.SVDQ_PROBE_FP6_DEQUANT])
def test_peak_probe_runs_and_is_deterministic(kind):
    """The benchmark's MFMA peak probe (include/svdq_probe.h): it launches,
    writes its whole sink, and two launches write the same bytes (the
    accumulations have a fixed order)."""
    blocks, iters = 64, 16
    per = 64
    sinks = []
    for _ in range(2):
        sink = torch.full((blocks * 256 * per + 256,), 0xA5, dtype=torch.uint8, device="cuda")
        L.check(L.lib().svdq_probe_mfma(kind, blocks, iters, sink.data_ptr(), torch.cuda.current_stream().cuda_stream),
                "probe")
        torch.cuda.synchronize()
        sinks.append(sink.cpu())
    assert torch.equal(sinks[0], sinks[1])
    assert torch.all(sinks[0][blocks * 256 * per:] == 0xA5)      # nothing written past the sink
    assert L.lib().svdq_probe_mfma_ops(kind, blocks, iters) > 0
