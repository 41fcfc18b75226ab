"""GPU parity of the INT4 layer on the 6-bit MFMA (codes in E3M2 containers)
against the CPU oracle, through the C ABI.

Bars as for the nibble kernels: codes, fp16 scales and the per-group integer
products bit-exact; lora_act within 1e-5 relative Frobenius; the bf16
output within 1e-3 relative Frobenius of the oracle's bf16 output, and
elementwise within one bf16 ulp of the oracle's value for all but a 1e-4
fraction of the elements.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from tests._fp6 import ACT, WGT, decode_fp6
from tests._helpers import (bf16_bits_to_f64, check_bf16_elementwise, f64_to_bf16_bits,  # noqa: F401
                            oracle_prep_to_abi, ulp_bf16)

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


def y_to_np(y):
    return y.double().cpu().numpy() if y.dtype == torch.float32 else to_np_bf16(y)


def pad_scales(sx_gm, M):
    """[G][M] scales -> the [G][32 ceil(M/32)] layout of the 6-bit path."""
    G = sx_gm.shape[0]
    Mp = 32 * ((M + 31) // 32)
    out = np.zeros((G, Mp), np.float16)
    out[:, :M] = sx_gm
    return out


def run_gemm(xf, xs, wf, ws, la, lu, bias, M, N, K, rank, out_dtype=L.SVDQ_OUT_BF16):
    y = S.gemm_w4a4_fp6_lora_up(xf, xs, wf, ws, la, lu, bias, M, N, K, rank, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


# ------------------------------------------------------------------ integer core
@pytest.mark.parametrize("M,N,K", [(300, 264, 256), (16, 128, 64), (129, 8, 128), (1, 136, 192),
                                   (200, 1032, 12288), (520, 776, 320), (4000, 4104, 320)])
def test_int32_group_products_bit_exact(M, N, K):
    """Unit scales, rank 0, fp32 output: y = sum_k q_x q_w is an integer below
    2^24, exact in fp32 in any order; bit for bit against the oracle's
    integer products, including -8 codes and the all -8 extreme P_g = 4096."""
    rng = np.random.default_rng(M * 7 + N + K)
    qx = rng.integers(-8, 8, (M, K))
    qw = rng.integers(-8, 8, (K, N))
    qx[0, :64] = -8
    qw[:64, 0] = -8
    G = K // 64
    ref = O.w4a4_product(qx, np.ones((M, G)), qw, np.ones((G, N)), 64)
    xf = dev(S.pack_fp6_operand(O.pack_int4(qx), ACT))
    wf = dev(S.pack_fp6_operand(O.pack_int4(qw.T), WGT))
    xs = dev(pad_scales(np.ones((G, M), np.float16), M))
    ws = dev(np.ones((G, N), np.float16))
    y = run_gemm(xf, xs, wf, ws, None, None, None, M, N, K, 0, L.SVDQ_OUT_F32)
    np.testing.assert_array_equal(y.double().cpu().numpy(), ref)


def test_int32_single_group_isolation():
    M, N, K = 64, 128, 512
    rng = np.random.default_rng(5)
    G = K // 64
    for g in (0, 3, 7):
        qx = np.zeros((M, K), np.int64)
        qw = np.zeros((K, N), np.int64)
        qx[:, 64 * g:64 * g + 64] = rng.integers(-8, 8, (M, 64))
        qw[64 * g:64 * g + 64] = rng.integers(-8, 8, (64, N))
        y = run_gemm(dev(S.pack_fp6_operand(O.pack_int4(qx), ACT)), dev(pad_scales(np.ones((G, M), np.float16), M)),
                     dev(S.pack_fp6_operand(O.pack_int4(qw.T), WGT)), dev(np.ones((G, N), np.float16)),
                     None, None, None, M, N, K, 0, L.SVDQ_OUT_F32)
        np.testing.assert_array_equal(y.double().cpu().numpy(), qx @ qw)


def test_dequant_scales_exact_fp32():
    """Power-of-two scales keep every product and sum exact in fp32 here,
    so the scaled result must equal the oracle's exactly: this pins which
    row scale and which column scale meet which tile element."""
    M, N, K = 96, 256, 256
    rng = np.random.default_rng(9)
    G = K // 64
    qx = rng.integers(-8, 8, (M, K))
    qw = rng.integers(-8, 8, (K, N))
    sx = np.exp2(rng.integers(-3, 4, (M, G))).astype(np.float16)
    sw = np.exp2(rng.integers(-3, 4, (G, N))).astype(np.float16)
    ref = O.w4a4_product(qx, sx.astype(np.float64), qw, sw.astype(np.float64), 64)
    y = run_gemm(dev(S.pack_fp6_operand(O.pack_int4(qx), ACT)), dev(pad_scales(sx.T, M)),
                 dev(S.pack_fp6_operand(O.pack_int4(qw.T), WGT)), dev(sw), None, None, None, M, N, K, 0,
                 L.SVDQ_OUT_F32)
    np.testing.assert_array_equal(y.double().cpu().numpy(), ref)


# ------------------------------------------------------------------ kernel 1
def _case(M, K, N, rank, seed, bias=False, n_out=4):
    wl = workloads.custom_workload(M, K, N, seed=seed, n_out=n_out, bias=bias)
    Lr = wl.layers[0]
    po = O.prepare(Lr.weight, wl.act_absmax(), rank=rank)
    return wl, Lr, po, oracle_prep_to_abi(po)


def run_k1(x_bits, smooth_inv, lora_down_bits, rank, act=L.SVDQ_ACT_NONE):
    xf, xs, la = S.quant_act_lora_down_fp6(dev_bf16(x_bits), dev(np.asarray(smooth_inv, np.float32)),
                                           dev_bf16(lora_down_bits) if rank else None, rank, act=act)
    torch.cuda.synchronize()
    return xf, xs, la


# (4200, 256, 32), at ranks 49-64 (8230, 192, 64) (more 32-row blocks than
# CUs: the 8-wave form) and, at ranks 65-128, (8200, 128, 128): enough rows
# for kernel 1's 32-row blocks; (4111, 192, 64) stays on 16-row blocks; odd
# M leaves padded rows
@pytest.mark.parametrize("M,K,rank", [(300, 512, 32), (1, 64, 16), (16, 128, 0), (257, 1024, 48),
                                      (64, 512, 128), (33, 256, 256), (77, 3072, 32), (40, 12288, 64),
                                      (1000, 1088, 16), (129, 2112, 256), (4200, 256, 32), (4111, 192, 64),
                                      (8230, 192, 64), (8200, 128, 128)])
def test_k1_codes_scales_lora_act(M, K, rank):
    N = max(64, ((rank + 7) // 8) * 8)
    wl, Lr, po, abi = _case(M, K, N, rank, seed=42 + M)
    x = wl.x.copy()
    x[M // 2] = 0.0
    xb = f64_to_bf16_bits(x)
    for rep in range(2):
        xf, xs, la = run_k1(xb, abi["smooth_inv"], abi["lora_down"], rank)
        q, s, xh = O.quantize_activation(x, po["smooth_inv"], 64)
        codes, pad = decode_fp6(xf.cpu().numpy(), M, K, ACT)
        np.testing.assert_array_equal(codes, q)
        assert np.all(pad == 0)
        xs_np = xs.cpu().numpy()
        np.testing.assert_array_equal(xs_np[:, :M].astype(np.float64), s.T)
        assert not xs_np[:, M:].any()
        if rank:
            ref = O.lora_down(xh, po["L1"])
            assert O.rel_fro(la.double().cpu().numpy(), ref) <= LORA_TOL


def test_k1_is_deterministic():
    M, K, rank = 300, 4096, 64
    wl, Lr, po, abi = _case(M, K, 64, rank, seed=3)
    xb = f64_to_bf16_bits(wl.x)
    outs = [run_k1(xb, abi["smooth_inv"], abi["lora_down"], rank)[2].cpu().numpy() for _ in range(3)]
    for o in outs[1:]:
        np.testing.assert_array_equal(o.view(np.uint32), outs[0].view(np.uint32))


def test_k1_matches_nibble_kernel():
    """Same codes and scales as the nibble kernel 1 on the same input."""
    M, K, rank = 513, 3072, 32
    wl, Lr, po, abi = _case(M, K, 128, rank, seed=8)
    xb = f64_to_bf16_bits(wl.x)
    xf, xs, la = run_k1(xb, abi["smooth_inv"], abi["lora_down"], rank)
    xc2, xs2, la2 = S.quant_act_lora_down(dev_bf16(xb), dev(abi["smooth_inv"]), dev_bf16(abi["lora_down"]), rank)
    torch.cuda.synchronize()
    codes, _ = decode_fp6(xf.cpu().numpy(), M, K, ACT)
    np.testing.assert_array_equal(codes, O.unpack_int4(xc2.cpu().numpy()))
    np.testing.assert_array_equal(xs.cpu().numpy()[:, :M], xs2.cpu().numpy())


@pytest.mark.parametrize("M,K,rank", [(256, 3072, 32), (4200, 512, 32), (8200, 256, 128)])
def test_k1_gelu_statistical(M, K, rank):
    """GELU on load: the device GELU and the oracle's fp64 tanh differ by a
    few ulps, so codes may differ at rounding boundaries (by 1, in at most
    1e-4 of them) and scales by at most one fp16 ulp.  (4200, 512, 32) and
    (8200, 256, 128) run kernel 1's 32-row blocks (more 16-row blocks than
    CUs)."""
    wl, Lr, po, abi = _case(M, K, max(64, rank), rank, seed=11)
    xb = f64_to_bf16_bits(wl.x)
    xf, xs, la = run_k1(xb, abi["smooth_inv"], abi["lora_down"], rank, act=L.SVDQ_ACT_GELU_TANH)
    q, s, xh = O.quantize_activation(wl.x, po["smooth_inv"], 64, act="gelu_tanh")
    codes, _ = decode_fp6(xf.cpu().numpy(), M, K, ACT)
    d = codes - q
    assert np.abs(d).max() <= 1 and np.count_nonzero(d) <= 1e-4 * d.size + 1
    sg = xs.cpu().numpy()[:, :M].astype(np.float64)
    assert np.all(np.abs(sg - s.T) <= np.abs(s.T) * 2.0 ** -10 + 1e-12)


# ------------------------------------------------------------------ whole layer
@pytest.mark.parametrize("M,K,N,rank,bias,out", [
    (300, 512, 264, 32, False, "bf16"), (300, 512, 264, 32, True, "f32"), (257, 1024, 520, 0, True, "bf16"),
    (64, 3072, 3072, 32, True, "bf16"), (1, 256, 136, 16, False, "bf16"), (513, 2048, 1032, 128, True, "bf16"),
    (520, 640, 776, 256, False, "f32"), (4000, 192, 4104, 48, True, "bf16")])
def test_forward_vs_oracle(M, K, N, rank, bias, out):
    wl, Lr, po, abi = _case(M, K, N, rank, seed=M + K + N, bias=bias)
    xb = f64_to_bf16_bits(wl.x)
    xf, xs, la = run_k1(xb, abi["smooth_inv"], abi["lora_down"], rank)
    wf = dev(S.pack_fp6_operand(abi["w_codes"], WGT))
    od = L.SVDQ_OUT_F32 if out == "f32" else L.SVDQ_OUT_BF16
    y = run_gemm(xf, xs, wf, dev(abi["w_scales"]), la, dev_bf16(abi["lora_up"]) if rank else None,
                 dev_bf16(Lr.bias_bits) if bias else None, M, N, K, rank, od)
    yg = y_to_np(y)
    yo = O.forward(wl.x, po, bias=Lr.bias if bias else None, out="f32" if out == "f32" else "bf16")
    err = O.rel_fro(yg, yo)
    if out == "f32":
        assert err <= 1e-5, err
    else:
        assert err <= Y_TOL, err
        check_bf16_elementwise(yg, yo)


def test_forward_matches_nibble_path():
    """With the same inputs, the 6-bit path and the int8 path add the same
    fp32 terms (identical codes, scales and exact group products); only the
    order of the fp32 sum differs (the int8 path's 128 x 128 form, used at
    this size, adds bias and up projection last), so their fp32 outputs agree
    within fp32 summation error."""
    M, K, N, rank = 512, 1024, 512, 32
    wl, Lr, po, abi = _case(M, K, N, rank, seed=21, bias=True)
    xb = f64_to_bf16_bits(wl.x)
    xf, xs, la = run_k1(xb, abi["smooth_inv"], abi["lora_down"], rank)
    y6 = run_gemm(xf, xs, dev(S.pack_fp6_operand(abi["w_codes"], WGT)), dev(abi["w_scales"]), la,
                  dev_bf16(abi["lora_up"]), dev_bf16(Lr.bias_bits), M, N, K, rank, L.SVDQ_OUT_F32)
    xc, xs2, la2 = S.quant_act_lora_down(dev_bf16(xb), dev(abi["smooth_inv"]), dev_bf16(abi["lora_down"]), rank)
    y8 = S.gemm_w4a4_lora_up(xc, xs2, dev(abi["w_codes"]), dev(abi["w_scales"]), la2, dev_bf16(abi["lora_up"]),
                             dev_bf16(Lr.bias_bits), M, N, K, rank, out_dtype=L.SVDQ_OUT_F32)
    torch.cuda.synchronize()
    assert O.rel_fro(y6.double().cpu().numpy(), y8.double().cpu().numpy()) <= 1e-5


def test_repeat_runs_bitwise_equal():
    M, K, N, rank = 600, 3072, 1024, 32
    wl, Lr, po, abi = _case(M, K, N, rank, seed=2, bias=True)
    xb = f64_to_bf16_bits(wl.x)
    wf = dev(S.pack_fp6_operand(abi["w_codes"], WGT))
    outs = []
    for _ in range(3):
        xf, xs, la = run_k1(xb, abi["smooth_inv"], abi["lora_down"], rank)
        outs.append(run_gemm(xf, xs, wf, dev(abi["w_scales"]), la, dev_bf16(abi["lora_up"]),
                             dev_bf16(Lr.bias_bits), M, N, K, rank).view(torch.int16).cpu().numpy())
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])
