"""Tail writes of every layer kernel: each output is placed inside a larger
device buffer whose guard bytes before and after it hold a canary pattern.
After the launch the guards are unchanged and the payload equals the oracle
(or, for the MXFP4 and AWQ variants, whose parity is tested elsewhere, the
same call's output in a plain buffer).  The shapes are ragged in M and N and
cover both tile forms of the nibble kernel 2 (128 x 128; 256 x 256 when M is
even and the grid holds at least 192 such tiles) and both block forms of
kernel 1 (16-row blocks; 32-row blocks once there are more 16-row blocks
than compute units)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from tests._fp6 import ACT, WGT, decode_fp6
from tests._helpers import (bf16_bits_to_f64, check_bf16_elementwise, check_f32_elementwise,
                            oracle_prep_to_abi)

S = pytest.importorskip("w4a4_rank_corrected_svdq_amd")
from w4a4_rank_corrected_svdq_amd import _lib as L  # noqa: E402

pytestmark = pytest.mark.gpu

GUARD = 4096
CANARY = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert S.device_check(0) == 0, "device is not gfx950"
    torch.cuda.set_device(0)


class Guarded:
    """A [shape] tensor of ``dtype`` at byte offset GUARD of a canary-filled
    buffer with GUARD spare bytes after it."""

    def __init__(self, shape, dtype):
        self.n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((2 * GUARD + self.n,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + self.n].view(dtype).view(shape)

    def check(self):
        b = self.buf.cpu().numpy()
        assert np.all(b[:GUARD] == CANARY), "write before the buffer"
        assert np.all(b[GUARD + self.n:] == CANARY), "write past the end of the buffer"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_np_bf16(t):
    return bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))


def _case(M, K, N, rank, seed, bias=True):
    wl = workloads.custom_workload(M, K, N, seed=seed, n_out=4, bias=bias)
    Lr = wl.layers[0]
    po = O.prepare(Lr.weight, wl.act_absmax(), rank=rank)
    return wl, Lr, po, oracle_prep_to_abi(po)


# 301 rows: 16-row blocks; 4111 rows: 32-row blocks (more 16-row blocks than CUs)
K1_CASES = [(301, 512, 32), (4111, 192, 64), (77, 256, 0)]


@pytest.mark.parametrize("M,K,rank", K1_CASES)
def test_k1_guarded(M, K, rank):
    wl, Lr, po, abi = _case(M, K, 64, rank, seed=90 + M)
    G = K // 64
    gc, gs = Guarded((M, K // 2), torch.uint8), Guarded((G, M), torch.float16)
    gl = Guarded((M, rank), torch.float32) if rank else None
    S.quant_act_lora_down(dev_bf16(wl.x_bits), dev(abi["smooth_inv"]),
                          dev_bf16(abi["lora_down"]) if rank else None, rank,
                          out=(gc.t, gs.t, gl.t if rank else None))
    torch.cuda.synchronize()
    for g in (gc, gs, gl):
        if g is not None:
            g.check()
    q, s, xh = O.quantize_activation(wl.x, po["smooth_inv"], 64)
    np.testing.assert_array_equal(gc.t.cpu().numpy(), O.pack_int4(q))
    np.testing.assert_array_equal(gs.t.cpu().numpy().astype(np.float64), s.T)
    if rank:
        assert O.rel_fro(gl.t.double().cpu().numpy(), O.lora_down(xh, po["L1"])) < 1e-5


# (301, 264): 128 x 128 form; (4000, 4104): 256 x 256 form, both ragged
K2_CASES = [(301, 512, 264, 32, "bf16"), (301, 512, 264, 16, "f32"),
            (4000, 192, 4104, 32, "bf16"), (4000, 128, 4104, 48, "f32"), (33, 64, 8, 0, "bf16")]


def _k2_inputs(M, K, N, rank, seed):
    wl, Lr, po, abi = _case(M, K, N, rank, seed)
    parts = O.forward(wl.x, po, bias=Lr.bias, out="f64", return_parts=True)[1]
    return wl, Lr, po, abi, parts


def _check_out(y, Yo_f64, out):
    if out == "f32":
        check_f32_elementwise(y.double().cpu().numpy(), O.fp32(Yo_f64))
    else:
        yb = to_np_bf16(y)
        assert O.rel_fro(yb, O.bf16(Yo_f64)) < 1e-3
        check_bf16_elementwise(yb, O.bf16(Yo_f64))


@pytest.mark.parametrize("M,K,N,rank,out", K2_CASES)
def test_k2_guarded(M, K, N, rank, out):
    wl, Lr, po, abi, parts = _k2_inputs(M, K, N, rank, seed=91 + M + rank)
    od = L.SVDQ_OUT_F32 if out == "f32" else L.SVDQ_OUT_BF16
    gy = Guarded((M, N), torch.float32 if out == "f32" else torch.bfloat16)
    S.gemm_w4a4_lora_up(dev(O.pack_int4(parts["qx"])), dev(parts["sx"].T.astype(np.float16)),
                        dev(abi["w_codes"]), dev(abi["w_scales"]),
                        dev(parts["lora_act"].astype(np.float32)) if rank else None,
                        dev_bf16(abi["lora_up"]) if rank else None, dev_bf16(Lr.bias_bits),
                        M, N, K, rank, out_dtype=od, out=gy.t)
    torch.cuda.synchronize()
    gy.check()
    _check_out(gy.t, parts["y"], out)


def test_qkv_guarded():
    M, K, heads, rank = 301, 256, 2, 16
    N = 3 * heads * 128
    wl, Lr, po, abi, parts = _k2_inputs(M, K, N, rank, seed=95)
    (qb, qv), (kb, kv) = workloads.norm_weights(seed=96)
    ang = np.random.default_rng(97).uniform(-np.pi, np.pi, (M, 64))
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    gy = Guarded((M, N), torch.bfloat16)
    S.gemm_w4a4_lora_up_qkv(dev(O.pack_int4(parts["qx"])), dev(parts["sx"].T.astype(np.float16)),
                            dev(abi["w_codes"]), dev(abi["w_scales"]), dev(parts["lora_act"].astype(np.float32)),
                            dev_bf16(abi["lora_up"]), dev_bf16(Lr.bias_bits), dev_bf16(qb), dev_bf16(kb),
                            dev(cos), dev(sin), M, N, K, rank, out=gy.t)
    torch.cuda.synchronize()
    gy.check()
    ref = O.forward_qkv(wl.x, po, Lr.bias, qv, kv, cos, sin)
    check_bf16_elementwise(to_np_bf16(gy.t), ref)


# ------------------------------------------------------------ 6-bit MFMA route
@pytest.mark.parametrize("M,K,rank", K1_CASES)
def test_k1_fp6_guarded(M, K, rank):
    wl, Lr, po, abi = _case(M, K, 64, rank, seed=98 + M)
    G, RB = K // 64, (M + 31) // 32
    gf, gs = Guarded((G, RB, 1536), torch.uint8), Guarded((G, 32 * RB), torch.float16)
    gl = Guarded((M, rank), torch.float32) if rank else None
    S.quant_act_lora_down_fp6(dev_bf16(wl.x_bits), dev(abi["smooth_inv"]),
                              dev_bf16(abi["lora_down"]) if rank else None, rank,
                              out=(gf.t, gs.t, gl.t if rank else None))
    torch.cuda.synchronize()
    for g in (gf, gs, gl):
        if g is not None:
            g.check()
    q, s, xh = O.quantize_activation(wl.x, po["smooth_inv"], 64)
    codes, pad = decode_fp6(gf.t.cpu().numpy(), M, K, ACT)
    np.testing.assert_array_equal(codes, q)
    assert np.all(pad == 0)
    xs = gs.t.cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(xs[:, :M], s.T)
    assert np.all(xs[:, M:] == 0)
    if rank:
        assert O.rel_fro(gl.t.double().cpu().numpy(), O.lora_down(xh, po["L1"])) < 1e-5


@pytest.mark.parametrize("M,K,N,rank,out", K2_CASES)
def test_k2_fp6_guarded(M, K, N, rank, out):
    wl, Lr, po, abi, parts = _k2_inputs(M, K, N, rank, seed=99 + M + rank)
    G, Mp = K // 64, 32 * ((M + 31) // 32)
    xs = np.zeros((G, Mp), np.float16)
    xs[:, :M] = parts["sx"].T
    od = L.SVDQ_OUT_F32 if out == "f32" else L.SVDQ_OUT_BF16
    gy = Guarded((M, N), torch.float32 if out == "f32" else torch.bfloat16)
    S.gemm_w4a4_fp6_lora_up(dev(S.pack_fp6_operand(O.pack_int4(parts["qx"]), ACT)), dev(xs),
                            dev(S.pack_fp6_operand(abi["w_codes"], WGT)), dev(abi["w_scales"]),
                            dev(parts["lora_act"].astype(np.float32)) if rank else None,
                            dev_bf16(abi["lora_up"]) if rank else None, dev_bf16(Lr.bias_bits),
                            M, N, K, rank, out_dtype=od, out=gy.t)
    torch.cuda.synchronize()
    gy.check()
    _check_out(gy.t, parts["y"], out)


@pytest.mark.parametrize("M,K,N,rank,out", [(300, 256, 384, 32, "bf16"), (4001, 128, 3072, 16, "bf16"),
                                             (129, 192, 576, 0, "f32")])
def test_k2_fp6_n192_guarded(M, K, N, rank, out):
    """The 256 x 192 form of the 6-bit kernel 2: ragged M (4001 rows leave
    the last tile row 161 deep), fp32 and bf16 outputs."""
    wl, Lr, po, abi, parts = _k2_inputs(M, K, N, rank, seed=131 + M + rank)
    G, Mp = K // 64, 32 * ((M + 31) // 32)
    xs = np.zeros((G, Mp), np.float16)
    xs[:, :M] = parts["sx"].T
    od = L.SVDQ_OUT_F32 if out == "f32" else L.SVDQ_OUT_BF16
    gy = Guarded((M, N), torch.float32 if out == "f32" else torch.bfloat16)
    S.gemm_w4a4_fp6_lora_up_n192(dev(S.pack_fp6_operand(O.pack_int4(parts["qx"]), ACT)), dev(xs),
                                 dev(S.pack_fp6_operand(abi["w_codes"], ACT)), dev(abi["w_scales"]),
                                 dev(parts["lora_act"].astype(np.float32)) if rank else None,
                                 dev_bf16(abi["lora_up"]) if rank else None, dev_bf16(Lr.bias_bits),
                                 M, N, K, rank, out_dtype=od, out=gy.t)
    torch.cuda.synchronize()
    gy.check()
    _check_out(gy.t, parts["y"], out)


# ------------------------------------------------------------ MXFP4 and AWQ
def test_mxfp4_guarded_equals_plain():
    M, K, N, rank = 301, 512, 264, 32
    wl = workloads.custom_workload(M, K, N, seed=100, n_out=4, bias=True)
    Lr = wl.layers[0]
    p = S.prepare_weights_mxfp4(Lr.weight_bits, wl.act_absmax(), rank=rank)
    x, si, ld = dev_bf16(wl.x_bits), dev(p["smooth_inv"]), dev_bf16(p["lora_down"])
    plain = S.quant_act_lora_down_mxfp4(x, si, ld, rank)
    g = (Guarded((M, K // 2), torch.uint8), Guarded((M, K // 32), torch.uint8), Guarded((M, rank), torch.float32))
    S.quant_act_lora_down_mxfp4(x, si, ld, rank, out=tuple(t.t for t in g))
    args = (dev(p["w_codes"]), dev(p["w_scales"]))
    y0 = S.gemm_mxfp4_lora_up(*plain[:2], *args, plain[2], dev_bf16(p["lora_up"]), dev_bf16(Lr.bias_bits),
                              M, N, K, rank)
    gy = Guarded((M, N), torch.bfloat16)
    S.gemm_mxfp4_lora_up(*plain[:2], *args, plain[2], dev_bf16(p["lora_up"]), dev_bf16(Lr.bias_bits),
                         M, N, K, rank, out=gy.t)
    torch.cuda.synchronize()
    for t in g + (gy,):
        t.check()
    for a, b in zip(plain, (t.t for t in g)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    assert torch.equal(y0.view(torch.int16), gy.t.view(torch.int16))


def test_awq_guarded_equals_plain():
    aw = workloads.awq_workload(5, K=576, N=416, Mc=8, seed=101)
    p = S.awq_prepare(aw["weight_bits"], aw["x_cal_bits"])
    M, K, N = 5, 576, 416
    x, inv = dev_bf16(aw["x_bits"]), dev(p["inv_scale"])
    xh, xs = S.awq_quant_act(x, inv)
    gh, gs = Guarded((M, K), torch.bfloat16), Guarded((K // 64, 16), torch.float32)
    S.awq_quant_act(x, inv, out=(gh.t, gs.t))
    w = (dev(p["w_codes"]), dev(p["w_scales"]), dev(p["w_zeros"]), dev_bf16(aw["bias_bits"]))
    y0 = S.awq_gemv(xh, xs, *w, M, N, K)
    gy = Guarded((M, N), torch.bfloat16)
    S.awq_gemv(xh, xs, *w, M, N, K, out=gy.t)
    torch.cuda.synchronize()
    for t in (gh, gs, gy):
        t.check()
    assert torch.equal(xh.view(torch.int16), gh.t.view(torch.int16))
    assert torch.equal(xs.view(torch.int32), gs.t.view(torch.int32))
    assert torch.equal(y0.view(torch.int16), gy.t.view(torch.int16))
