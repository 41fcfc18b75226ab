"""The no-allocation MLP-chain entry point (svdq_gemm_w4a4_fp6_mlp_chain_noalloc)
through the C ABI: two calls in a row, the second smaller, each bit for bit
equal to the workspace entry point on the same inputs; a request whose
partials exceed the device scratch is refused before any device work."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from tests._fp6 import WGT

S = pytest.importorskip("w4a4_rank_corrected_svdq_amd")
from w4a4_rank_corrected_svdq_amd import _lib as L  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert S.device_check(0) == 0, "device is not gfx950"
    torch.cuda.set_device(0)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(M, K, N, N2, r, seed):
    wl = workloads.custom_workload(M, K, N, seed=seed, n_out=4, bias=True, second_N=N2)
    up, dn = wl.layers
    bf = lambda b: torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16)  # noqa: E731
    lu = S.SVDQW4A4Linear(S.prepare_weights(up.weight_bits, wl.act_absmax(), rank=r), bf(up.bias_bits), "cuda")
    x = torch.from_numpy(wl.x_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    y_up = lu(x)
    a_dn = torch.nn.functional.gelu(y_up.float(), approximate="tanh").abs().amax(0).cpu().numpy()
    ld = S.SVDQW4A4Linear(S.prepare_weights(dn.weight_bits, a_dn, rank=r), bf(dn.bias_bits), "cuda")
    xf, xs, la = S.quant_act_lora_down_fp6(x, lu.smooth_inv, lu.lora_down, r)
    return lu, ld, xf, xs, la, M, N, K, r


def _outputs(M, N, r):
    RB = (M + 31) // 32
    return (torch.full((N // 64, RB, 1536), 0x5A, dtype=torch.uint8, device="cuda"),
            torch.full((N // 64, 32 * RB), 7.0, dtype=torch.float16, device="cuda"),
            torch.full((M, r), -3.0, dtype=torch.float32, device="cuda"))


def _noalloc(lu, ld, xf, xs, la, M, N, K, r, out):
    st = L.lib().svdq_gemm_w4a4_fp6_mlp_chain_noalloc(
        xf.data_ptr(), xs.data_ptr(), lu.w_fp6.data_ptr(), lu.w_scales.data_ptr(), la.data_ptr(),
        lu.lora_up.data_ptr(), lu.bias.data_ptr(), M, N, K, r, 64, ld.smooth_inv.data_ptr(),
        ld.lora_down.data_ptr(), r, out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    L.check(st, "svdq_gemm_w4a4_fp6_mlp_chain_noalloc")


def test_noalloc_matches_workspace_entry_two_calls():
    for M, K, N, N2, r, seed in ((300, 256, 768, 192, 32, 5), (64, 128, 256, 128, 16, 6)):
        lu, ld, xf, xs, la, M, N, K, r = _case(M, K, N, N2, r, seed)
        ref = S.gemm_w4a4_fp6_mlp_chain(xf, xs, lu.w_fp6, lu.w_scales, la, lu.lora_up, lu.bias, M, N, K, r,
                                        ld.smooth_inv, ld.lora_down, r)
        out = _outputs(M, N, r)
        _noalloc(lu, ld, xf, xs, la, M, N, K, r, out)
        torch.cuda.synchronize()
        assert torch.equal(out[0], ref[0])
        assert torch.equal(out[1].view(torch.int16), ref[1].view(torch.int16))
        assert torch.equal(out[2].view(torch.int32), ref[2].view(torch.int32))


def test_noalloc_refuses_requests_beyond_its_scratch():
    # 48 column slices x 65536 rows x 16 ranks x 4 bytes = 192 MiB of partials
    M, N, K, r = 65536, 12288, 64, 16
    t = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    p = t.data_ptr()
    need = ctypes.c_size_t(0)
    L.lib().svdq_mlp_chain_workspace_bytes(M, N, r, ctypes.byref(need))
    assert need.value > L.SVDQ_CHAIN_SCRATCH_BYTES
    st = L.lib().svdq_gemm_w4a4_fp6_mlp_chain_noalloc(p, p, p, p, p, p, None, M, N, K, r, 64, p, p, r, p, p, p, None)
    assert st == L.SVDQ_ERR_UNSUPPORTED_SHAPE
