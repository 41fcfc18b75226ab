"""GPU parity of the AWQ W4A16 path (through the C ABI) against the AWQ oracle.

Bars: x_hat bit-exact; xsum equal to the fp32 sum in increasing k; output
within 1e-3 relative Frobenius of the oracle's bf16 output (the inner sums
run on bf16 MFMA with fp32 accumulation; the oracle sums in fp64), and
elementwise within one bf16 ulp plus the first-order bound of the kernel's
fp32 rounding (see ``fp32_allowance``).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from oracle import awq_oracle as A
from tests._helpers import bf16_bits_to_f64, check_bf16_elementwise

S = pytest.importorskip("w4a4_rank_corrected_svdq_amd")

pytestmark = pytest.mark.gpu

Y_TOL = 1e-3


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


def _pack(q):
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def _case(M, K, N, seed, alpha=None):
    wl = workloads.awq_workload(M, K=K, N=N, Mc=16, seed=seed)
    po = A.awq_prepare(wl["weight"], wl["x_cal"], alpha=alpha)
    return wl, po


def _run(wl, po, bias=True):
    M, K, N = wl["M"], wl["K"], wl["N"]
    xh, xs = S.awq_quant_act(dev_bf16(wl["x_bits"]), dev(po["inv_scale"].astype(np.float32)))
    y = S.awq_gemv(xh, xs, dev(_pack(po["q"])), dev(po["s"].astype(np.float16)), dev(po["z"].astype(np.uint8)),
                   dev_bf16(wl["bias_bits"]) if bias else None, M, N, K)
    torch.cuda.synchronize()
    return xh, xs, y


def fp32_allowance(x_hat, po, bias):
    """First-order worst-case rounding of the kernel's fp32 sums, n u sum|t|,
    for the form it evaluates: sum_g s_g (sum_k (128 + q) x_hat - (128 + z_g)
    X_g) + bias, whose terms are about 128 times larger than the result, so
    that a small output can move by more than one bf16 ulp.  n = 4 product
    blocks per group + G groups + 8 wave partials + 2 (scale and bias) for
    the MFMA forms; the single-row form (M = 1) rounds each term at most
    4 (dot-product chain) + 2 + 1 (lane pair) + 1 (zero point) + K/2048
    (chunks) + 5 (lane tree) + 1 (bias) times, never more than that n."""
    M, K = x_hat.shape
    G = K // 64
    ax = np.abs(x_hat)
    t1 = ax @ ((128.0 + po["q"]) * np.repeat(po["s"], 64, axis=1)).T
    t2 = ax.reshape(M, G, 64).sum(-1) @ (po["s"] * (128.0 + po["z"])).T
    mag = t1 + t2 + (0.0 if bias is None else np.abs(bias)[None, :])
    return (4 + G + 8 + 2) * 2.0 ** -24 * mag


@pytest.mark.parametrize("M,K", [(1, 512), (5, 3072), (16, 192)])
def test_awq_quant_act_exact(M, K):
    wl, po = _case(M, K, 32, seed=60 + M, alpha=0.5)
    xh, xs, _ = _run(wl, po)
    x_hat = O.bf16(O.fp32(wl["x"] * po["inv_scale"][None, :]))
    np.testing.assert_array_equal(to_np_bf16(xh), x_hat)
    sums = np.zeros((K // 64, 16), np.float32)
    for g in range(K // 64):
        sums[g, :M] = np.cumsum(x_hat[:, 64 * g:64 * g + 64].astype(np.float32), axis=1, dtype=np.float32)[:, -1]
    np.testing.assert_array_equal(xs.cpu().numpy(), sums)


@pytest.mark.parametrize("M,K,N,bias", [(1, 512, 288, True), (3, 3072, 128, True), (16, 1024, 64, False),
                                        (7, 64, 32, True), (2, 4160, 96, False), (9, 8192, 64, True)])
def test_awq_gemv_parity(M, K, N, bias):
    wl, po = _case(M, K, N, seed=70 + M + K)
    _, _, y = _run(wl, po, bias)
    ref = A.awq_forward(wl["x"], po, bias=wl["bias"] if bias else None)
    assert O.rel_fro(to_np_bf16(y), ref) < Y_TOL
    x_hat = O.bf16(O.fp32(wl["x"] * po["inv_scale"][None, :]))
    check_bf16_elementwise(to_np_bf16(y), ref, atol=fp32_allowance(x_hat, po, wl["bias"] if bias else None))


@pytest.mark.parametrize("K,N,bias", [(64, 32, True), (512, 288, True), (2048, 96, False), (3072, 18432, True),
                                      (4160, 64, True), (8192, 32, False)])
def test_awq_linear_row_equals_two_kernels(K, N, bias):
    """svdq_awq_linear_row (one row, scaling and GEMV in one launch) against
    svdq_awq_quant_act + svdq_awq_gemv at M = 1: bit for bit (one, two,
    three and four 1 KB code chunks per row; N not a multiple of a block's
    24 channels), and against the oracle."""
    wl, po = _case(1, K, N, seed=90 + K // 64 + N)
    xh, xs, y2 = _run(wl, po, bias)
    y1 = S.awq_linear_row(dev_bf16(wl["x_bits"]), dev(po["inv_scale"].astype(np.float32)), dev(_pack(po["q"])),
                          dev(po["s"].astype(np.float16)), dev(po["z"].astype(np.uint8)),
                          dev_bf16(wl["bias_bits"]) if bias else None, N, K)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    ref = A.awq_forward(wl["x"], po, bias=wl["bias"] if bias else None)
    x_hat = O.bf16(O.fp32(wl["x"] * po["inv_scale"][None, :]))
    check_bf16_elementwise(to_np_bf16(y1), ref, atol=fp32_allowance(x_hat, po, wl["bias"] if bias else None))


def test_awq_linear_row_argument_errors():
    import ctypes
    from w4a4_rank_corrected_svdq_amd import _lib as L
    t = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(t.data_ptr())
    fn = L.lib().svdq_awq_linear_row
    assert fn(p, p, p, p, p, None, 64, 8256, p, None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE   # K past the row form
    assert fn(p, p, p, p, p, None, 48, 128, p, None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE    # N % 32
    assert fn(p, p, p, p, p, None, 64, 96, p, None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE     # K % 64
    assert fn(None, p, p, p, p, None, 64, 128, p, None) == L.SVDQ_ERR_INVALID_ARG
    assert fn(p, p, p, p, p, None, 0, 128, p, None) == L.SVDQ_ERR_INVALID_ARG


@pytest.mark.parametrize("M", [1, 2])
def test_awq_full_size_modulation(M):
    """FLUX double-block modulation projection 3072 -> 18432 with bias, the
    benchmark's launch configuration; the whole output against the oracle."""
    wl, po = _case(M, 3072, 18432, seed=80 + M)
    _, _, y = _run(wl, po)
    ref = A.awq_forward(wl["x"], po, bias=wl["bias"])
    assert O.rel_fro(to_np_bf16(y), ref) < Y_TOL
    x_hat = O.bf16(O.fp32(wl["x"] * po["inv_scale"][None, :]))
    check_bf16_elementwise(to_np_bf16(y), ref, atol=fp32_allowance(x_hat, po, wl["bias"]))
    assert torch.isfinite(y.float()).all()


def test_awq_module_and_error_story():
    """Library-prepared layer: the searched alpha beats plain round-to-nearest
    (alpha = 0) against fp64 x W^T, measured on the GPU output."""
    wl = workloads.awq_workload(16, K=1024, N=512, Mc=32, seed=90)
    ref = wl["x"] @ wl["weight"].T + wl["bias"][None, :]
    lin = torch.nn.Linear(1024, 512, bias=True)
    with torch.no_grad():
        lin.weight.copy_(torch.from_numpy(wl["weight"]))
        lin.bias.copy_(torch.from_numpy(wl["bias"]))
    x = dev_bf16(wl["x_bits"])
    xc = torch.from_numpy(wl["x_cal_bits"].view(np.int16).copy()).view(torch.bfloat16)
    errs = {}
    for alpha in (-1.0, 0.0):
        m = S.AWQW4A16Linear.from_linear(lin, xc, alpha=alpha)
        errs[alpha] = O.rel_fro(to_np_bf16(m(x)), ref)
    assert errs[-1.0] < errs[0.0] < 0.1, errs
