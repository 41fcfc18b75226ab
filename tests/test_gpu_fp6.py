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
from tests._helpers import (bf16_bits_to_f64, check_bf16_elementwise, check_f32_elementwise, f64_to_bf16_bits,  # noqa: F401,E501
                            abi_to_oracle_prep, check_int4_codes_in_band, oracle_prep_to_abi, ulp_bf16)

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
def test_k1_gelu_codes_in_band(M, K, rank):
    """GELU on load: the device GELU and the oracle's fp64 tanh differ by
    ~1e-6 relative, so a scale or code may differ only where the oracle's
    value lies that close to its rounding boundary (then either candidate is
    valid); everywhere else they are equal.  (4200, 512, 32) and
    (8200, 256, 128) run kernel 1's 32-row blocks (more 16-row blocks than
    CUs)."""
    wl, Lr, po, abi = _case(M, K, max(64, rank), rank, seed=11)
    xb = f64_to_bf16_bits(wl.x)
    xf, xs, la = run_k1(xb, abi["smooth_inv"], abi["lora_down"], rank, act=L.SVDQ_ACT_GELU_TANH)
    q, s, xh = O.quantize_activation(wl.x, po["smooth_inv"], 64, act="gelu_tanh")
    codes, _ = decode_fp6(xf.cpu().numpy(), M, K, ACT)
    amb_s, amb_q = check_int4_codes_in_band(codes, xs.cpu().numpy()[:, :M].astype(np.float64).T, xh)
    assert amb_s <= 0.03 * s.size and amb_q <= 1e-4 * q.size   # the band is narrow


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


# ------------------------------------------------------------------ fused QKV epilogue
def _check(yg, yo, out):
    """The output bars of this file: 1e-3 relative Frobenius and one bf16 ulp
    elementwise (bf16), or 1e-5 and 2^-14 (|y| + rms y) elementwise (fp32)."""
    err = O.rel_fro(yg, yo)
    if out == "f32":
        assert err <= 1e-5, err
        check_f32_elementwise(yg, yo)
    else:
        assert err <= Y_TOL, err
        check_bf16_elementwise(yg, yo)


def _qkv_tables(M, seed, rope):
    (qb, qv), (kb, kv) = workloads.norm_weights(seed=seed)
    cos = sin = None
    if rope:
        ang = np.random.default_rng(seed).uniform(-np.pi, np.pi, (M, 64))
        cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    return qb, qv, kb, kv, cos, sin


def run_qkv6(xf, xs, wf, abi, la, bias_bits, M, qb, kb, cos, sin, out_dtype=L.SVDQ_OUT_BF16):
    r = abi["rank"]
    y = S.gemm_w4a4_fp6_lora_up_qkv(xf, xs, wf, dev(abi["w_scales"]), la, dev_bf16(abi["lora_up"]) if r else None,
                                    dev_bf16(bias_bits) if bias_bits is not None else None,
                                    dev_bf16(qb), dev_bf16(kb),
                                    dev(cos) if cos is not None else None, dev(sin) if sin is not None else None,
                                    M, abi["N"], abi["K"], r, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


# heads = 3 puts the Q / K boundary inside a 256-column tile (its first wave
# Q, its second K); 11 heads on M = 4000 leave the last tile column half past
# N and the last tile row 160 rows deep (rotary rows past M read as zeros and
# never stored); M = 1 is a single row.  K = 64 and 128 (two stages per tile)
# and K = 256 at rank 16 (three) put the staged rotary factors into ring
# slots that the first stages use.
@pytest.mark.parametrize("M,K,heads,rank,bias,rope,out", [
    (300, 512, 2, 32, True, True, "bf16"), (300, 512, 2, 32, True, True, "f32"), (64, 512, 1, 0, False, False, "bf16"),
    (129, 512, 3, 16, True, False, "f32"), (513, 512, 3, 32, True, True, "bf16"), (1, 512, 1, 16, True, True, "bf16"),
    (4000, 256, 11, 16, True, True, "bf16"), (200, 64, 2, 0, True, True, "bf16"), (300, 128, 3, 16, False, True, "f32"),
    (520, 256, 1, 16, True, True, "bf16")])
def test_qkv_epilogue_vs_oracle(M, K, heads, rank, bias, rope, out):
    """The 6-bit kernel 2 with the fused QKV epilogue (per-head RMSNorm of Q
    and K, rotary embedding of their adjacent pairs) against the oracle's
    fused QKV operator on the oracle's own codes, scales and lora_act; the V
    columns bit-identical to the plain 6-bit kernel."""
    N = 3 * heads * 128
    wl, Lr, po, abi = _case(M, K, N, rank, seed=70 + M + heads, bias=bias)
    qb, qv, kb, kv, cos, sin = _qkv_tables(M, 71 + M, rope)
    _, parts = O.forward(wl.x, po, bias=Lr.bias if bias else None, out="f64", return_parts=True)
    ref = O.forward_qkv(wl.x, po, Lr.bias if bias else None, qv, kv, cos, sin, out=out)
    xf = dev(S.pack_fp6_operand(O.pack_int4(parts["qx"]), ACT))
    xs = dev(pad_scales(parts["sx"].T.astype(np.float16), M))
    wf = dev(S.pack_fp6_operand(abi["w_codes"], WGT))
    la = dev(parts["lora_act"].astype(np.float32)) if rank else None
    od = L.SVDQ_OUT_F32 if out == "f32" else L.SVDQ_OUT_BF16
    bb = Lr.bias_bits if bias else None
    y = run_qkv6(xf, xs, wf, abi, la, bb, M, qb, kb, cos, sin, out_dtype=od)
    _check(y_to_np(y), ref, out)
    plain = run_gemm(xf, xs, wf, dev(abi["w_scales"]), la, dev_bf16(abi["lora_up"]) if rank else None,
                     dev_bf16(bb) if bb is not None else None, M, N, K, rank, od)
    v0 = 2 * heads * 128
    np.testing.assert_array_equal(y[:, v0:].view(torch.int16 if out == "bf16" else torch.int32).cpu().numpy(),
                                  plain[:, v0:].view(torch.int16 if out == "bf16" else torch.int32).cpu().numpy())


def test_qkv_full_size_sampled_rows():
    """The joint-stream QKV shape (4096 image + 512 text rows, 3072 -> 9216,
    rank 32, bias) with rotary tables of the FLUX form, through both 6-bit
    kernels in the launch configuration the benchmark times: sampled rows
    (first, last, random) against the oracle's fused QKV operator, every V
    column bit-identical to the plain 6-bit kernel."""
    wl = workloads.make_workload("joint_qkv")
    Lr = wl.layers[0]
    M, K, N, r = wl.M, Lr.K, Lr.N, 32
    rng = np.random.default_rng(13)
    a = wl.act_absmax()
    _, lam = O.smoothing_factors(a, Lr.weight)
    l1 = O.bf16(rng.standard_normal((K, r)) * float(np.abs(lam).mean() * 0.02))
    l2 = O.bf16(rng.standard_normal((r, N)) / np.sqrt(N))
    po = O.prepare(Lr.weight, a, rank=r, factors=(l1, l2))
    abi = oracle_prep_to_abi(po)
    (qb, qv), (kb, kv) = workloads.norm_weights(seed=14)
    cos, sin = workloads.rope_tables(512, 64)
    xf, xs, la = run_k1(wl.x_bits, abi["smooth_inv"], abi["lora_down"], r)
    wf = dev(S.pack_fp6_operand(abi["w_codes"], WGT))
    y = run_qkv6(xf, xs, wf, abi, la, Lr.bias_bits, M, qb, kb, cos, sin)
    rows = np.unique(np.concatenate([np.arange(8), rng.choice(M, 32, replace=False), np.arange(M - 8, M)]))
    ref = O.forward_qkv(wl.x[rows], po, Lr.bias, qv, kv, cos[rows], sin[rows])
    _check(to_np_bf16(y[torch.from_numpy(rows).cuda()]), ref, "bf16")
    assert torch.isfinite(y.float()).all()
    plain = run_gemm(xf, xs, wf, dev(abi["w_scales"]), la, dev_bf16(abi["lora_up"]), dev_bf16(Lr.bias_bits),
                     M, N, K, r)
    v0 = 2 * N // 3
    assert torch.equal(y[:, v0:].view(torch.int16), plain[:, v0:].view(torch.int16))


@pytest.mark.parametrize("engine", ["fp6", "int8"])
def test_linear_forward_qkv(engine):
    """SVDQW4A4Linear.forward_qkv (its own kernel 1, then the fused QKV
    kernel 2 of the engine) against the oracle's fused QKV operator on the
    library-prepared arrays; its V columns equal the module's plain forward."""
    M, K, heads, r = 300, 512, 2, 32
    N = 3 * heads * 128
    wl = workloads.custom_workload(M, K, N, seed=83, n_out=4, bias=True)
    Lr = wl.layers[0]
    p = S.prepare_weights(Lr.weight_bits, wl.act_absmax(), rank=r)
    po = abi_to_oracle_prep(p)
    # auto_route off: the plain forward stays on the engine's own kernels, so
    # its V columns are the fused kernel's bit for bit
    lin = S.SVDQW4A4Linear(p, torch.from_numpy(Lr.bias_bits.view(np.int16).copy()).view(torch.bfloat16), "cuda",
                           engine=engine, auto_route=False)
    qb, qv, kb, kv, cos, sin = _qkv_tables(M, 84, True)
    x = dev_bf16(wl.x_bits)
    y = lin.forward_qkv(x, dev_bf16(qb), dev_bf16(kb), dev(cos), dev(sin))
    plain = lin(x)
    torch.cuda.synchronize()
    _check(to_np_bf16(y), O.forward_qkv(wl.x, po, Lr.bias, qv, kv, cos, sin), "bf16")
    v0 = 2 * heads * 128
    assert torch.equal(y[:, v0:].view(torch.int16), plain[:, v0:].view(torch.int16))


# ------------------------------------------------------------------ 256 x 192 tile form
def run_n192(xf, xs, wr, ws, la, lu, bias, M, N, K, rank, out_dtype=L.SVDQ_OUT_BF16):
    y = S.gemm_w4a4_fp6_lora_up_n192(xf, xs, wr, ws, la, lu, bias, M, N, K, rank, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M,N,K", [(300, 192, 256), (16, 384, 64), (1, 192, 192), (520, 576, 320),
                                   (4000, 768, 320), (200, 1152, 12288), (257, 3072, 128)])
def test_n192_int32_group_products_bit_exact(M, N, K):
    """The 256 x 192 form with unit scales, rank 0, fp32 output: bit for bit
    the oracle's integer products (-8 extremes included), so the transposed
    operand roles and the plain row-block weight layout meet every (token,
    channel) pair exactly once."""
    rng = np.random.default_rng(M * 11 + N + K)
    qx = rng.integers(-8, 8, (M, K))
    qw = rng.integers(-8, 8, (K, N))
    qx[0, :64] = -8
    qw[:64, 0] = -8
    G = K // 64
    ref = O.w4a4_product(qx, np.ones((M, G)), qw, np.ones((G, N)), 64)
    y = run_n192(dev(S.pack_fp6_operand(O.pack_int4(qx), ACT)), dev(pad_scales(np.ones((G, M), np.float16), M)),
                 dev(S.pack_fp6_operand(O.pack_int4(qw.T), ACT)), dev(np.ones((G, N), np.float16)),
                 None, None, None, M, N, K, 0, L.SVDQ_OUT_F32)
    np.testing.assert_array_equal(y.double().cpu().numpy(), ref)


def test_n192_dequant_scales_exact_fp32():
    """Power-of-two scales keep every product and sum exact in fp32: the
    scaled result equals the oracle's exactly, which pins which token scale
    and which channel scale meet which element in the transposed form."""
    M, N, K = 96, 384, 256
    rng = np.random.default_rng(19)
    G = K // 64
    qx = rng.integers(-8, 8, (M, K))
    qw = rng.integers(-8, 8, (K, N))
    sx = np.exp2(rng.integers(-3, 4, (M, G))).astype(np.float16)
    sw = np.exp2(rng.integers(-3, 4, (G, N))).astype(np.float16)
    ref = O.w4a4_product(qx, sx.astype(np.float64), qw, sw.astype(np.float64), 64)
    y = run_n192(dev(S.pack_fp6_operand(O.pack_int4(qx), ACT)), dev(pad_scales(sx.T, M)),
                 dev(S.pack_fp6_operand(O.pack_int4(qw.T), ACT)), dev(sw), None, None, None, M, N, K, 0,
                 L.SVDQ_OUT_F32)
    np.testing.assert_array_equal(y.double().cpu().numpy(), ref)


@pytest.mark.parametrize("M,K,N,rank,bias,out", [
    (300, 512, 192, 32, False, "bf16"), (300, 512, 384, 32, True, "f32"), (257, 1024, 576, 0, True, "bf16"),
    (64, 3072, 3072, 32, True, "bf16"), (1, 256, 192, 16, False, "bf16"), (513, 2048, 1152, 128, True, "bf16"),
    (520, 640, 768, 256, False, "f32"), (4000, 192, 3072, 48, True, "bf16")])
def test_n192_forward_vs_oracle(M, K, N, rank, bias, out):
    """Kernel 1 then the 256 x 192 form against the oracle's forward: ranks
    0 to 256, ragged M, bias, bf16 and fp32 outputs."""
    wl, Lr, po, abi = _case(M, K, N, rank, seed=M + K + N + 5, bias=bias)
    xb = f64_to_bf16_bits(wl.x)
    xf, xs, la = run_k1(xb, abi["smooth_inv"], abi["lora_down"], rank)
    wr = dev(S.pack_fp6_operand(abi["w_codes"], ACT))
    od = L.SVDQ_OUT_F32 if out == "f32" else L.SVDQ_OUT_BF16
    y = run_n192(xf, xs, wr, dev(abi["w_scales"]), la, dev_bf16(abi["lora_up"]) if rank else None,
                 dev_bf16(Lr.bias_bits) if bias else None, M, N, K, rank, od)
    yo = O.forward(wl.x, po, bias=Lr.bias if bias else None, out="f32" if out == "f32" else "bf16")
    _check(y_to_np(y), yo, out)


def test_n192_matches_256_form():
    """Both tile forms add the same exact group products with the same two
    scales, each group rounded once (the 256 x 256 form scales by s_x first,
    the 256 x 192 form by s_w first), so their fp32 outputs agree within
    fp32 summation error."""
    M, K, N, rank = 512, 1024, 768, 32
    wl, Lr, po, abi = _case(M, K, N, rank, seed=23, bias=True)
    xf, xs, la = run_k1(f64_to_bf16_bits(wl.x), abi["smooth_inv"], abi["lora_down"], rank)
    args = (dev(abi["w_scales"]), la, dev_bf16(abi["lora_up"]), dev_bf16(Lr.bias_bits), M, N, K, rank,
            L.SVDQ_OUT_F32)
    y192 = run_n192(xf, xs, dev(S.pack_fp6_operand(abi["w_codes"], ACT)), *args)
    y256 = run_gemm(xf, xs, dev(S.pack_fp6_operand(abi["w_codes"], WGT)), *args)
    assert O.rel_fro(y192.double().cpu().numpy(), y256.double().cpu().numpy()) <= 1e-6


def test_n192_full_size_attention_out_sampled_rows():
    """The attention output projection (4096 x 3072 -> 3072, rank 32, bias)
    through the module, which takes the 256 x 192 form on a 256-CU device
    (256 tiles against 192 of 256 x 256): sampled rows (first, last, random)
    against the oracle, repeat runs bitwise equal."""
    wl = workloads.make_workload("attn_out")
    Lr = wl.layers[0]
    M, K, N, r = wl.M, Lr.K, Lr.N, 32
    rng = np.random.default_rng(17)
    a = wl.act_absmax()
    _, lam = O.smoothing_factors(a, Lr.weight)
    l1 = O.bf16(rng.standard_normal((K, r)) * float(np.abs(lam).mean() * 0.02))
    l2 = O.bf16(rng.standard_normal((r, N)) / np.sqrt(N))
    po = O.prepare(Lr.weight, a, rank=r, factors=(l1, l2))
    abi = oracle_prep_to_abi(po)
    prep = dict(smooth_inv=abi["smooth_inv"], w_codes=abi["w_codes"], w_scales=abi["w_scales"],
                lora_down=abi["lora_down"], lora_up=abi["lora_up"], rank=r, group=64, K=K, N=N)
    bias = torch.from_numpy(Lr.bias_bits.view(np.int16).copy()).view(torch.bfloat16) if Lr.bias_bits is not None \
        else None
    lin = S.SVDQW4A4Linear(prep, bias, "cuda")
    assert lin.w_fp6_rows is not None
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert S.fp6_n192_preferred(M, N) and not S.fp6_n192_preferred(M, 12288)
    x = dev_bf16(wl.x_bits)
    y = lin(x)
    y2 = lin(x)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    rows = np.unique(np.concatenate([np.arange(8), rng.choice(M, 32, replace=False), np.arange(M - 8, M)]))
    ref = O.forward(wl.x[rows], po, bias=Lr.bias)
    _check(to_np_bf16(y[torch.from_numpy(rows).cuda()]), ref, "bf16")


def test_n192_copy_optional():
    """n192=False keeps no plain-layout copy and runs the 256 x 256 form:
    the same output as with the copy within fp32 summation order (both forms
    against each other at bf16: within one ulp)."""
    M, K, N, rank = 300, 512, 384, 32
    wl = workloads.custom_workload(M, K, N, seed=91, n_out=4, bias=True)
    Lr = wl.layers[0]
    p = S.prepare_weights(Lr.weight_bits, wl.act_absmax(), rank=rank)
    bias = torch.from_numpy(Lr.bias_bits.view(np.int16).copy()).view(torch.bfloat16)
    a = S.SVDQW4A4Linear(p, bias, "cuda", auto_route=False)
    b = S.SVDQW4A4Linear(p, bias, "cuda", n192=False, auto_route=False)
    assert a.w_fp6_rows is not None and b.w_fp6_rows is None
    x = dev_bf16(wl.x_bits)
    ya, yb = a(x), b(x)
    torch.cuda.synchronize()
    check_bf16_elementwise(to_np_bf16(ya), to_np_bf16(yb), frac=0.0)


def test_empty_batch_launches_nothing():
    """M = 0 (an empty batch) through every kernel entry point of the INT4
    layer: status OK and no byte of the (canary-filled) outputs written."""
    K, N, r = 128, 384, 16
    dev_u8 = lambda n: torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")  # noqa: E731
    b = [dev_u8(1 << 16) for _ in range(12)]
    p = [t.data_ptr() for t in b]
    st = torch.cuda.current_stream().cuda_stream
    lib = L.lib()
    calls = {
        "quant_act_lora_down": lib.svdq_quant_act_lora_down(p[0], p[1], p[2], 0, K, r, 64, 0, p[3], p[4], p[5], st),
        "quant_act_lora_down_fp6": lib.svdq_quant_act_lora_down_fp6(p[0], p[1], p[2], 0, K, r, 64, 0, p[3], p[4],
                                                                    p[5], st),
        "gemm_w4a4_lora_up": lib.svdq_gemm_w4a4_lora_up(p[0], p[1], p[2], p[3], p[4], p[5], None, 0, N, K, r, 64, 0,
                                                        p[6], st),
        "gemm_w4a4_fp6_lora_up": lib.svdq_gemm_w4a4_fp6_lora_up(p[0], p[1], p[2], p[3], p[4], p[5], None, 0, N, K, r,
                                                                64, 0, p[6], st),
        "gemm_w4a4_fp6_lora_up_n192": lib.svdq_gemm_w4a4_fp6_lora_up_n192(p[0], p[1], p[2], p[3], p[4], p[5], None, 0,
                                                                          N, K, r, 64, 0, p[6], st),
        "gemm_w4a4_lora_up_qkv": lib.svdq_gemm_w4a4_lora_up_qkv(p[0], p[1], p[2], p[3], p[4], p[5], None, p[7], p[8],
                                                                None, None, 1e-6, 0, N, K, r, 64, 0, p[6], st),
        "gemm_w4a4_fp6_lora_up_qkv": lib.svdq_gemm_w4a4_fp6_lora_up_qkv(p[0], p[1], p[2], p[3], p[4], p[5], None,
                                                                        p[7], p[8], p[9], p[10], 1e-6, 0, N, K, r, 64,
                                                                        0, p[6], st),
    }
    torch.cuda.synchronize()
    assert all(v == 0 for v in calls.values()), calls
    for t in b:
        assert bool((t == 0xA5).all())


@pytest.mark.parametrize("M,K,N", [(256, 512, 512), (1024, 3072, 3072), (4096, 256, 3072), (2048, 256, 12288)])
def test_int4_route(M, K, N):
    """A 6-bit layer's forward() runs the int8 engine's kernels where 256-row
    tiles would cover fewer than half the CUs (svdq_int4_route == 2) and the
    6-bit kernels otherwise; either way the output matches the oracle, and
    with auto_route off it matches the 6-bit kernels' own output within one
    bf16 ulp (fp32 sums in another order)."""
    wl = workloads.custom_workload(M, K, N, seed=97, n_out=4, bias=True)
    Lr = wl.layers[0]
    p = S.prepare_weights(Lr.weight_bits, wl.act_absmax(), rank=32)
    bias = torch.from_numpy(Lr.bias_bits.view(np.int16).copy()).view(torch.bfloat16)
    lin = S.SVDQW4A4Linear(p, bias, "cuda")
    fixed = S.SVDQW4A4Linear(p, bias, "cuda", auto_route=False)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    small = 2 * ((M + 255) // 256) * ((N + 255) // 256) < cus
    assert (S.int4_route(M, N) == 2) == small
    assert lin.route(M) == ("int8" if small else "fp6") and fixed.route(M) == "fp6"
    x = dev_bf16(wl.x_bits)
    y, y6 = lin(x), fixed(x)
    torch.cuda.synchronize()
    _check(to_np_bf16(y), O.forward(wl.x, abi_to_oracle_prep(p), bias=Lr.bias), "bf16")
    check_bf16_elementwise(to_np_bf16(y), to_np_bf16(y6), frac=1e-4)
