"""The MLP chain (svdq_gemm_w4a4_fp6_mlp_chain): the up layer's 6-bit
kernel 2 with the down layer's kernel 1 in its epilogue.

Bars: the down layer's codes and scales bit for bit equal to what the
two-layer path writes on the GPU (kernel 2 of the up layer, then kernel 1 of
the down layer with tanh-GELU, the same arithmetic); lora_act within 1e-5
relative Frobenius of the two-layer path's (the chain sums per-slice fp32
partials); the down layer's output against the oracle's chain within 1e-3
relative Frobenius, and elementwise within one bf16 ulp of the oracle's
kernel-2 arithmetic on the chain's own kernel-1 outputs (tanh-GELU codes may
sit on a rounding boundary, so codes are compared with the oracle
statistically); guard bytes around every output unchanged.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from tests._fp6 import ACT, WGT, decode_fp6
from tests._helpers import bf16_bits_to_f64, check_bf16_elementwise, f64_to_bf16_bits, oracle_prep_to_abi

S = pytest.importorskip("w4a4_rank_corrected_svdq_amd")
from w4a4_rank_corrected_svdq_amd import _lib as L  # noqa: E402

pytestmark = pytest.mark.gpu

GUARD, CANARY = 4096, 0xA5


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


class Guarded:
    def __init__(self, shape, dtype):
        self.n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((2 * GUARD + self.n,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + self.n].view(dtype).view(shape)

    def check(self):
        b = self.buf.cpu().numpy()
        assert np.all(b[:GUARD] == CANARY) and np.all(b[GUARD + self.n:] == CANARY)


def _pair(M, K, N, N2, r_up, r_dn, seed, synthetic=False):
    wl = workloads.custom_workload(M, K, N, seed=seed, n_out=4, bias=True, second_N=N2)
    up, dn = wl.layers
    rng = np.random.default_rng(seed)
    a_up = wl.act_absmax()
    if synthetic:
        # seeded bf16 factors: no full-size SVD in the oracle's preparation
        def fac(Lr, a, r):
            _, lam = O.smoothing_factors(a, Lr.weight)
            return (O.bf16(rng.standard_normal((Lr.K, r)) * float(np.abs(lam).mean() * 0.02)),
                    O.bf16(rng.standard_normal((r, Lr.N)) / np.sqrt(Lr.N)))
        pu = O.prepare(up.weight, a_up, rank=r_up, factors=fac(up, a_up, r_up) if r_up else None)
    else:
        pu = O.prepare(up.weight, a_up, rank=r_up)
    y_up = O.forward(wl.x, pu, bias=up.bias)
    a_dn = np.abs(O.gelu_tanh(y_up)).max(0).astype(np.float32)
    if synthetic:
        pd = O.prepare(dn.weight, a_dn, rank=r_dn, factors=fac(dn, a_dn, r_dn) if r_dn else None)
    else:
        pd = O.prepare(dn.weight, a_dn, rank=r_dn)
    return wl, up, dn, pu, pd


def _up_inputs(wl, up, pu):
    au = oracle_prep_to_abi(pu)
    r = au["rank"]
    x = dev_bf16(wl.x_bits)
    xf, xs, la = S.quant_act_lora_down_fp6(x, dev(au["smooth_inv"]), dev_bf16(au["lora_down"]) if r else None, r)
    wf = dev(S.pack_fp6_operand(au["w_codes"], WGT))
    return au, xf, xs, la, wf


def run_two_layer(wl, up, dn, pu, pd):
    """Kernel 2 of the up layer writes Y; kernel 1 of the down layer (GELU)
    reads it."""
    au, xf, xs, la, wf = _up_inputs(wl, up, pu)
    ad = oracle_prep_to_abi(pd)
    M, N, K = wl.M, up.N, up.K
    y_up = S.gemm_w4a4_fp6_lora_up(xf, xs, wf, dev(au["w_scales"]), la, dev_bf16(au["lora_up"]) if au["rank"] else None,
                                   dev_bf16(up.bias_bits), M, N, K, au["rank"])
    out = S.quant_act_lora_down_fp6(y_up, dev(ad["smooth_inv"]), dev_bf16(ad["lora_down"]) if ad["rank"] else None,
                                    ad["rank"], act=L.SVDQ_ACT_GELU_TANH)
    torch.cuda.synchronize()
    return out, y_up


def run_chain(wl, up, dn, pu, pd, guarded=False):
    au, xf, xs, la, wf = _up_inputs(wl, up, pu)
    ad = oracle_prep_to_abi(pd)
    M, N, K, rd = wl.M, up.N, up.K, ad["rank"]
    RB = (M + 31) // 32
    g = None
    if guarded:
        g = (Guarded((N // 64, RB, 1536), torch.uint8), Guarded((N // 64, 32 * RB), torch.float16),
             Guarded((M, rd), torch.float32) if rd else None)
    out = S.gemm_w4a4_fp6_mlp_chain(
        xf, xs, wf, dev(au["w_scales"]), la, dev_bf16(au["lora_up"]) if au["rank"] else None, dev_bf16(up.bias_bits),
        M, N, K, au["rank"], dev(ad["smooth_inv"]), dev_bf16(ad["lora_down"]) if rd else None, rd,
        out=None if g is None else (g[0].t, g[1].t, g[2].t if rd else None))
    torch.cuda.synchronize()
    if g is not None:
        for x in g:
            if x is not None:
                x.check()
    return out, ad


def run_down(xf, xs, la, ad, dn, M):
    wf = dev(S.pack_fp6_operand(ad["w_codes"], WGT))
    r = ad["rank"]
    y = S.gemm_w4a4_fp6_lora_up(xf, xs, wf, dev(ad["w_scales"]), la, dev_bf16(ad["lora_up"]) if r else None,
                                dev_bf16(dn.bias_bits), M, dn.N, dn.K, r)
    torch.cuda.synchronize()
    return y


def _down_from_codes(xf, xs, la, pd, bias, M, rows=None):
    """The oracle's kernel-2 arithmetic on given kernel-1 outputs."""
    K = pd["qw"].shape[0]
    q, _ = decode_fp6(xf.cpu().numpy(), M, K, ACT)
    sx = xs.cpu().numpy().astype(np.float64)[:, :M].T
    rows = slice(None) if rows is None else rows
    y = O.w4a4_product(q[rows], sx[rows], pd["qw"], pd["sw"], 64)
    if pd["L1"].shape[1]:
        y = y + O.bf16(la.double().cpu().numpy()[rows]) @ pd["L2"]
    return O.bf16(y + np.asarray(bias, np.float64)[None, :])


@pytest.mark.parametrize("M,K,N,N2,r_up,r_dn", [(300, 256, 512, 192, 32, 16), (64, 128, 256, 128, 16, 32),
                                                (33, 192, 576, 64, 0, 48), (257, 64, 320, 136, 16, 0)])
def test_chain_matches_two_layer_path_and_oracle(M, K, N, N2, r_up, r_dn):
    wl, up, dn, pu, pd = _pair(M, K, N, N2, r_up, r_dn, seed=M + N)
    (xf2, xs2, la2), _ = run_two_layer(wl, up, dn, pu, pd)
    (xf, xs, la), ad = run_chain(wl, up, dn, pu, pd, guarded=True)
    np.testing.assert_array_equal(xf.cpu().numpy(), xf2.cpu().numpy())
    np.testing.assert_array_equal(xs.cpu().numpy(), xs2.cpu().numpy())
    if r_dn:
        assert O.rel_fro(la.double().cpu().numpy(), la2.double().cpu().numpy()) <= 1e-5
    y = run_down(xf, xs, la, ad, dn, M)
    Yo, parts = O.forward_mlp_chain(wl.x, pu, pd, up.bias, dn.bias, return_parts=True)
    assert O.rel_fro(to_np_bf16(y), Yo) < 1e-3
    check_bf16_elementwise(to_np_bf16(y), _down_from_codes(xf, xs, la, pd, dn.bias, M))
    q, _ = decode_fp6(xf.cpu().numpy(), M, N, ACT)
    mism = q != parts["qx"]
    assert mism.mean() <= 1e-3 and np.all(np.abs(q - parts["qx"])[mism] == 1)
    if r_dn:
        assert O.rel_fro(la.double().cpu().numpy(), parts["lora_act"]) < 1e-4


def test_chain_module_and_repeat_runs():
    """SVDQMLPChain (library-prepared layers) against the two-layer modules
    on the 6-bit kernels (auto_route off: at this M their forward would take
    the int8 engine's kernels), and two calls bit-identical (fixed reduction
    order)."""
    M, K, N, N2 = 200, 256, 512, 256
    wl = workloads.custom_workload(M, K, N, seed=77, n_out=4, bias=True, second_N=N2)
    up, dn = wl.layers
    bf = lambda b: torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16)  # noqa: E731
    lu = S.SVDQW4A4Linear(S.prepare_weights(up.weight_bits, wl.act_absmax(), rank=32), bf(up.bias_bits), "cuda",
                          auto_route=False)
    x = dev_bf16(wl.x_bits)
    y_up = lu(x)
    a_dn = torch.nn.functional.gelu(y_up.float(), approximate="tanh").abs().amax(0).cpu().numpy()
    ld = S.SVDQW4A4Linear(S.prepare_weights(dn.weight_bits, a_dn, rank=32), bf(dn.bias_bits), "cuda",
                          auto_route=False)
    two = ld(y_up, act=L.SVDQ_ACT_GELU_TANH)
    chain = S.SVDQMLPChain(lu, ld)
    y1, y2 = chain(x), chain(x)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert O.rel_fro(to_np_bf16(y1), to_np_bf16(two)) < 1e-4
    with pytest.raises(ValueError):
        S.SVDQMLPChain(lu, lu)          # the down layer's K (256) is not the up layer's N (512)


def test_chain_argument_errors():
    M, K, N = 64, 128, 256
    t = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    p = t.data_ptr()
    ch = L.lib().svdq_gemm_w4a4_fp6_mlp_chain
    assert ch(p, p, p, p, p, p, None, M, 264, K, 16, 64, p, p, 16, p, p, p, p, 1 << 20, None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert ch(p, p, p, p, p, p, None, M, N, K, 16, 64, p, p, 16, p, p, p, p, 16, None) == L.SVDQ_ERR_INVALID_ARG
    assert ch(p, p, p, p, p, p, None, M, N, K, 16, 64, p, p, 24, p, p, p, p, 1 << 20, None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert ch(p, p, p, p, p, p, None, M, N, K, 16, 64, p, None, 16, p, p, p, p, 1 << 20, None) == L.SVDQ_ERR_INVALID_ARG


def test_chain_full_size_mlp_pair():
    """The FLUX MLP pair, 4096 x 3072 -> 12288 -> 3072, rank 32 on both
    layers: every code and scale of the down layer's input bit for bit
    against the two-layer path, lora_act within 1e-5, the down layer's output
    against the oracle's chain on sampled rows."""
    M, K, N, N2 = 4096, 3072, 12288, 3072
    wl, up, dn, pu, pd = _pair(M, K, N, N2, 32, 32, seed=3, synthetic=True)
    (xf2, xs2, la2), _ = run_two_layer(wl, up, dn, pu, pd)
    (xf, xs, la), ad = run_chain(wl, up, dn, pu, pd)
    assert torch.equal(xf, xf2) and torch.equal(xs.view(torch.int16), xs2.view(torch.int16))
    assert O.rel_fro(la.double().cpu().numpy(), la2.double().cpu().numpy()) <= 1e-5
    del xf2, xs2, la2
    y = run_down(xf, xs, la, ad, dn, M)
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([np.arange(4), rng.choice(M, 24, replace=False), np.arange(M - 4, M)]))
    Yo = O.forward_mlp_chain(wl.x[rows], pu, pd, up.bias, dn.bias)
    yr = to_np_bf16(y[torch.from_numpy(rows).cuda()])
    assert O.rel_fro(yr, Yo) < 1e-3
    check_bf16_elementwise(yr, _down_from_codes(xf, xs, la, pd, dn.bias, M, rows))
