"""CPU tests of the C ABI library: symbols, argument validation, the device
refusal path, and host preparation against the oracle."""
import ctypes
import glob
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import oracle as O
import workloads
from tests._helpers import bf16_bits_to_f64, f64_to_bf16_bits

S = pytest.importorskip("w4a4_rank_corrected_svdq_amd")
from w4a4_rank_corrected_svdq_amd import _lib as L  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(svdq_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 8
    h = L.lib()
    for n in names:
        assert hasattr(h, n), n
    assert set(names) == set(L.SIGNATURES)
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\sT {n}$", out, re.M), n


def test_status_strings():
    for st in range(-5, 1):
        assert L.status_string(st).startswith("SVDQ_")
    assert "UNKNOWN" in L.status_string(-99)


@pytest.mark.parametrize("K,N,rank,group,expect", [
    (3072, 12288, 32, 64, L.SVDQ_OK),
    (0, 64, 0, 64, L.SVDQ_ERR_INVALID_ARG),
    (128, 64, 80, 64, L.SVDQ_ERR_INVALID_ARG),        # rank > N
    (128, 64, -16, 64, L.SVDQ_ERR_INVALID_ARG),
    (96, 64, 16, 64, L.SVDQ_ERR_UNSUPPORTED_SHAPE),   # K % 64
    (128, 60, 16, 64, L.SVDQ_ERR_UNSUPPORTED_SHAPE),  # N % 8
    (128, 64, 24, 64, L.SVDQ_ERR_UNSUPPORTED_SHAPE),  # rank % 16
    (128, 64, 16, 32, L.SVDQ_ERR_UNSUPPORTED_SHAPE),  # group != 64
    (1024, 1024, 272, 64, L.SVDQ_ERR_UNSUPPORTED_SHAPE),  # rank > 256
])
def test_prepared_bytes_validation(K, N, rank, group, expect):
    out = ctypes.c_size_t(0)
    assert L.lib().svdq_prepared_bytes(K, N, rank, group, ctypes.byref(out)) == expect
    if expect == L.SVDQ_OK:
        assert out.value == O.prepared_bytes(K, N, rank, group)


def _fake(n=1):
    # 16-byte aligned host addresses; never dereferenced (validation fails first)
    buf = (ctypes.c_uint8 * 4096)()
    base = (ctypes.addressof(buf) + 15) & ~15
    return buf, [base + 256 * i for i in range(n)]


def test_device_entry_validation_precedes_device_use():
    buf, p = _fake(10)
    q = L.lib().svdq_quant_act_lora_down
    g = L.lib().svdq_gemm_w4a4_lora_up
    # invalid arguments are reported before any device query
    assert q(p[0], p[1], p[2], 16, 96, 32, 64, 0, p[3], p[4], p[5], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert q(None, p[1], p[2], 16, 128, 32, 64, 0, p[3], p[4], p[5], None) == L.SVDQ_ERR_INVALID_ARG
    assert q(p[0], p[1], None, 16, 128, 32, 64, 0, p[3], p[4], p[5], None) == L.SVDQ_ERR_INVALID_ARG
    assert q(p[0], p[1], p[2], 16, 128, 32, 64, 7, p[3], p[4], p[5], None) == L.SVDQ_ERR_INVALID_ARG
    assert q(p[0] + 2, p[1], p[2], 16, 128, 32, 64, 0, p[3], p[4], p[5], None) == L.SVDQ_ERR_INVALID_ARG
    assert q(p[0], p[1], p[2], -1, 128, 32, 64, 0, p[3], p[4], p[5], None) == L.SVDQ_ERR_INVALID_ARG
    assert g(p[0], p[1], p[2], p[3], p[4], p[5], None, 16, 64, 128, 32, 64, 0, None, None) == L.SVDQ_ERR_INVALID_ARG
    assert g(p[0], p[1], p[2], p[3], p[4], p[5], None, 16, 60, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert g(p[0], p[1], p[2], p[3], p[4], p[5], None, 16, 64, 128, 16, 64, 2, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    assert g(p[0], p[1], p[2], p[3], None, None, None, 16, 64, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    assert g(p[0], p[1], p[2], p[3], p[4], p[5], p[7] + 8, 16, 64, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    qk = L.lib().svdq_gemm_w4a4_lora_up_qkv
    #        xc    xs    wc    ws    la    lu    bias  nq    nk    cos   sin   eps   M   N    K    r   g   out y
    assert qk(p[0], p[1], p[2], p[3], p[4], p[5], None, p[6], p[7], p[8], p[9], 1e-6, 16, 256, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert qk(p[0], p[1], p[2], p[3], p[4], p[5], None, None, p[7], p[8], p[9], 1e-6, 16, 384, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    assert qk(p[0], p[1], p[2], p[3], p[4], p[5], None, p[6], p[7], p[8], None, 1e-6, 16, 384, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    assert qk(p[0], p[1], p[2], p[3], p[4], p[5], None, p[6], p[7], p[8], p[9], -1.0, 16, 384, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    assert qk(p[0], p[1], p[2], p[3], p[4], p[5], None, p[6], p[7] + 2, None, None, 1e-6, 16, 384, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    # rotary tables of 2 GiB or more (M * 256 bytes) are refused before any device use
    big = (1 << 23) + 16
    assert qk(p[0], p[1], p[2], p[3], p[4], p[5], None, p[6], p[7], p[8], p[9], 1e-6, big, 384, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    # the 6-bit kernel 2 addresses y and lora_act with 32-bit offsets: an
    # output of 2 GiB or more is refused before any device use
    g6 = L.lib().svdq_gemm_w4a4_fp6_lora_up
    #       x6    xs    w6    ws    la    lu    bias  M        N      K    r   g   out y
    assert g6(p[0], p[1], p[2], p[3], p[4], p[5], None, 1 << 17, 8192, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert g6(p[0], p[1], p[2], p[3], p[4], p[5], None, 1 << 16, 8192, 128, 16, 64, 1, p[6], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    n6 = L.lib().svdq_gemm_w4a4_fp6_lora_up_n192
    #       x6    xs    w6    ws    la    lu    bias  M        N      K    r   g   out y
    assert n6(p[0], p[1], p[2], p[3], p[4], p[5], None, 16, 256, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert n6(p[0], p[1], p[2], p[3], p[4], p[5], None, 16, 384, 96, 16, 64, 0, p[6], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert n6(p[0], p[1], None, p[3], p[4], p[5], None, 16, 384, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    assert n6(p[0], p[1], p[2], p[3], p[4], p[5], None, 16, 384, 128, 16, 64, 3, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    assert n6(p[0], p[1], p[2], p[3] + 4, p[4], p[5], None, 16, 384, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    assert n6(p[0], p[1], p[2], p[3], p[4], p[5], None, 1 << 17, 8448, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    q6 = L.lib().svdq_gemm_w4a4_fp6_lora_up_qkv
    #       x6    xs    w6    ws    la    lu    bias  nq    nk    cos   sin   eps   M   N    K    r   g   out y
    assert q6(p[0], p[1], p[2], p[3], p[4], p[5], None, p[6], p[7], p[8], p[9], 1e-6, 16, 256, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert q6(p[0], p[1], p[2], p[3], p[4], p[5], None, p[6], None, p[8], p[9], 1e-6, 16, 384, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    assert q6(p[0], p[1], p[2], p[3], p[4], p[5], None, p[6], p[7], None, p[9], 1e-6, 16, 384, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    assert q6(p[0], p[1], p[2], p[3], p[4], p[5], None, p[6], p[7], p[8], p[9], float("nan"), 16, 384, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    assert q6(p[0], p[1], p[2], p[3], p[4], p[5], None, p[6] + 2, p[7], None, None, 1e-6, 16, 384, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_INVALID_ARG
    assert q6(p[0], p[1], p[2], p[3], p[4], p[5], None, p[6], p[7], p[8], p[9], 1e-6, big, 384, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert q6(p[0], p[1], p[2], p[3], p[4], p[5], None, p[6], p[7], None, None, 1e-6, 1 << 17, 8448, 128, 16, 64, 0, p[6], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    pr = L.lib().svdq_probe_mfma
    assert pr(5, 1, 1, p[0], None) == L.SVDQ_ERR_INVALID_ARG          # unknown kind
    assert pr(-1, 1, 1, p[0], None) == L.SVDQ_ERR_INVALID_ARG
    assert pr(0, 0, 1, p[0], None) == L.SVDQ_ERR_INVALID_ARG          # no blocks
    assert pr(1, 1, 0, p[0], None) == L.SVDQ_ERR_INVALID_ARG          # no iterations
    assert pr(0, 1, 1, p[0] + 4, None) == L.SVDQ_ERR_INVALID_ARG      # misaligned sink
    ops = L.lib().svdq_probe_mfma_ops
    assert ops(0, 3, 5) == 3 * 4 * 5 * 1 * 2 * 32 * 32 * 32
    assert ops(1, 3, 5) == 3 * 4 * 5 * 4 * 2 * 32 * 32 * 64
    assert ops(L.SVDQ_PROBE_MFMA_FP6, 3, 5) == ops(L.SVDQ_PROBE_FP6_DEQUANT, 3, 5) == 3 * 4 * 5 * 8 * 2 * 32 * 32 * 64
    assert ops(L.SVDQ_PROBE_DEQUANT, 3, 5) == 3 * 4 * 5 * 8 * 3 * 32 * 32
    assert ops(7, 3, 5) == 0.0
    d = L.lib().svdq_lora_down
    u = L.lib().svdq_lora_up_add
    assert d(p[0], p[1], p[2], 16, 128, 0, 64, 0, p[3], None) == L.SVDQ_ERR_INVALID_ARG       # rank 0
    assert d(p[0], p[1], p[2], 16, 128, 24, 64, 0, p[3], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert d(p[0], p[1], p[2], 16, 96, 32, 64, 0, p[3], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert d(p[0], p[1], p[2], 16, 32768 + 64, 32, 64, 0, p[3], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert d(p[0], p[1], None, 16, 128, 32, 64, 0, p[3], None) == L.SVDQ_ERR_INVALID_ARG
    assert d(p[0], p[1], p[2], 16, 128, 32, 64, 3, p[3], None) == L.SVDQ_ERR_INVALID_ARG
    assert d(p[0], p[1], p[2], 16, 128, 32, 64, 0, p[3] + 4, None) == L.SVDQ_ERR_INVALID_ARG
    assert u(p[0], p[1], 16, 128, 0, p[2], None) == L.SVDQ_ERR_INVALID_ARG                    # rank 0
    assert u(p[0], p[1], 16, 100, 16, p[2], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert u(p[0], p[1], 16, 128, 24, p[2], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert u(p[0], p[1], 16, 16, 32, p[2], None) == L.SVDQ_ERR_INVALID_ARG                    # rank > N
    assert u(p[0], None, 16, 128, 16, p[2], None) == L.SVDQ_ERR_INVALID_ARG
    assert u(p[0], p[1], -1, 128, 16, p[2], None) == L.SVDQ_ERR_INVALID_ARG


REFUSAL_SCRIPT = r"""
import ctypes, sys
sys.path.insert(0, {root!r})
from w4a4_rank_corrected_svdq_amd import _lib as L
buf = (ctypes.c_uint8 * 4096)()
b = (ctypes.addressof(buf) + 15) & ~15
p = [b + 256 * i for i in range(8)]
r1 = L.lib().svdq_quant_act_lora_down(p[0], p[1], p[2], 16, 128, 32, 64, 0, p[3], p[4], p[5], None)
r2 = L.lib().svdq_gemm_w4a4_lora_up(p[0], p[1], p[2], p[3], p[4], p[5], None, 16, 64, 128, 16, 64, 0, p[6], None)
r3 = L.lib().svdq_device_check(0)
r4 = L.lib().svdq_lora_down(p[0], p[1], p[2], 16, 128, 32, 64, 0, p[3], None)
r5 = L.lib().svdq_lora_up_add(p[0], p[1], 16, 128, 16, p[2], None)
r6 = L.lib().svdq_quant_act_lora_down_mxfp4(p[0], p[1], p[2], 16, 128, 32, 0, p[3], p[4], p[5], None)
r7 = L.lib().svdq_gemm_mxfp4_lora_up(p[0], p[1], p[2], p[3], p[4], p[5], None, 16, 64, 128, 16, 0, p[6], None)
r8 = L.lib().svdq_gemm_w4a4_lora_up_qkv(p[0], p[1], p[2], p[3], p[4], p[5], None, p[6], p[7], None, None, 1e-6,
                                        16, 384, 128, 16, 64, 0, p[6], None)
print(r1, r2, r3, r4, r5, r6, r7, r8)
"""


def test_unsupported_device_is_refused():
    """A non-gfx950 device (forced through SVDQ_ASSUME_ARCH) or no device at
    all gives SVDQ_ERR_UNSUPPORTED_DEVICE and launches nothing ("Hardware
    support": refuse with a clear error rather than compute wrong results)."""
    env = dict(os.environ, SVDQ_ASSUME_ARCH="gfx942:sramecc+:xnack-")
    r = subprocess.run([sys.executable, "-c", REFUSAL_SCRIPT.format(root=ROOT)], env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == [str(L.SVDQ_ERR_UNSUPPORTED_DEVICE)] * 8


# ------------------------------------------------------------ host preparation
def _bits(v):
    return f64_to_bf16_bits(v)


@pytest.mark.parametrize("shape", [(256, 512, 512), (64, 256, 136)])
def test_prepare_rank0_bit_exact(shape):
    M, K, N = shape
    wl = workloads.custom_workload(M, K, N, seed=31, n_out=4)
    Lr = wl.layers[0]
    p = S.prepare_weights(Lr.weight_bits, wl.act_absmax(), rank=0)
    po = O.prepare(Lr.weight, wl.act_absmax(), rank=0)
    np.testing.assert_array_equal(p["smooth_inv"].astype(np.float64), po["smooth_inv"])
    np.testing.assert_array_equal(p["w_codes"], O.pack_int4(po["qw"].T))
    np.testing.assert_array_equal(p["w_scales"].astype(np.float64), po["sw"])


@pytest.mark.parametrize("alpha", [0.25, 0.75])
def test_prepare_other_alpha(alpha):
    wl = workloads.custom_workload(64, 256, 64, seed=32)
    p = S.prepare_weights(wl.layers[0].weight_bits, wl.act_absmax(), rank=0, alpha=alpha)
    si, _ = O.smoothing_factors(wl.act_absmax(), wl.layers[0].weight, alpha=alpha)
    np.testing.assert_allclose(p["smooth_inv"].astype(np.float64), si, rtol=2 ** -23)


@pytest.mark.parametrize("rank", [16, 32, 48])
def test_prepare_given_factors_bit_exact(rank):
    """Given the oracle's bf16 factors, residual codes and scales match bit for bit."""
    wl = workloads.custom_workload(128, 512, 384, seed=33, n_out=6)
    Lr = wl.layers[0]
    po = O.prepare(Lr.weight, wl.act_absmax(), rank=rank)
    p = S.prepare_weights(Lr.weight_bits, wl.act_absmax(), rank=rank,
                          factors=(_bits(po["L1"].T), _bits(po["L2"].T)))
    np.testing.assert_array_equal(p["w_codes"], O.pack_int4(po["qw"].T))
    np.testing.assert_array_equal(p["w_scales"].astype(np.float64), po["sw"])
    np.testing.assert_array_equal(p["lora_down"], _bits(po["L1"].T))


@pytest.mark.parametrize("shape,rank", [((256, 512, 512), 32), ((64, 384, 1024), 64), ((64, 256, 128), 128)])
def test_prepare_svd_accuracy(shape, rank):
    """The library's own top-r split: outlier singular values match LAPACK,
    the bf16 residual is within 0.5% of the oracle's (Eckart-Young optimum up
    to bf16 rounding), and the product L1 L2 spans the same top subspace."""
    M, K, N = shape
    wl = workloads.custom_workload(M, K, N, seed=34, n_out=4)
    Lr = wl.layers[0]
    p = S.prepare_weights(Lr.weight_bits, wl.act_absmax(), rank=rank, return_sigma=True)
    po = O.prepare(Lr.weight, wl.act_absmax(), rank=rank)
    sig = po["sigma"]
    np.testing.assert_allclose(p["sigma"][:4], sig[:4], rtol=1e-9)
    assert np.all(np.abs(p["sigma"] / sig[:rank] - 1) < 0.05)
    l1 = bf16_bits_to_f64(p["lora_down"]).T
    l2 = bf16_bits_to_f64(p["lora_up"]).T
    res_lib = np.linalg.norm(po["W_hat"] - l1 @ l2)
    res_orc = np.linalg.norm(po["W_hat"] - po["L1"] @ po["L2"])
    opt = np.sqrt((sig[rank:] ** 2).sum())
    assert res_orc >= opt * (1 - 1e-12)
    assert res_lib <= res_orc * 1.005
    # codes are self-consistent: same residual quantizer as the oracle
    R = po["W_hat"] - l1 @ l2
    q, s = O.quantize_weight_residual(R, 64)
    assert np.mean(O.pack_int4(q.T) == p["w_codes"]) > 0.9999
    np.testing.assert_array_equal(p["w_scales"].astype(np.float64), s)


def test_prepare_full_rank_zero_residual():
    wl = workloads.custom_workload(32, 128, 64, seed=35)
    Lr = wl.layers[0]
    p = S.prepare_weights(Lr.weight_bits, wl.act_absmax(), rank=64, return_sigma=True)
    po = O.prepare(Lr.weight, wl.act_absmax(), rank=64, round_factors=False)
    np.testing.assert_allclose(p["sigma"], po["sigma"][:64], rtol=1e-9)
    # only bf16 rounding of the factors is left in the residual
    l1 = bf16_bits_to_f64(p["lora_down"]).T
    l2 = bf16_bits_to_f64(p["lora_up"]).T
    assert O.rel_fro(l1 @ l2, po["W_hat"]) < 2 ** -7


def test_prepare_numeric_errors():
    K, N = 128, 64
    w = np.zeros((N, K), np.uint16)
    a = np.ones(K, np.float32)
    w[3, 5] = 0x7F80  # +inf
    with pytest.raises(S.SVDQError) as e:
        S.prepare_weights(w, a, rank=0)
    assert e.value.status == L.SVDQ_ERR_NUMERIC
    w[3, 5] = 0
    a[7] = np.nan
    with pytest.raises(S.SVDQError) as e:
        S.prepare_weights(w, a, rank=0)
    assert e.value.status == L.SVDQ_ERR_NUMERIC
    # fp16 scale overflow: |R| / 7 above 65504 after smoothing by lambda = 1
    w2 = np.full((N, K), f64_to_bf16_bits(O.bf16(np.array([1e6])))[0], np.uint16)
    with pytest.raises(S.SVDQError) as e:
        S.prepare_weights(w2, np.full(K, 1e6, np.float32), rank=0)
    assert e.value.status == L.SVDQ_ERR_NUMERIC


def test_prepare_zero_weight():
    K, N = 128, 64
    p = S.prepare_weights(np.zeros((N, K), np.uint16), np.zeros(K, np.float32), rank=16)
    assert np.all(p["w_codes"] == 0) and np.all(p["w_scales"] == 0)


def test_binding_rejects_non_contiguous_host_arrays():
    from w4a4_rank_corrected_svdq_amd import ops
    w = np.zeros((128, 64), np.uint16).T          # F-ordered [64][128]
    with pytest.raises(TypeError):
        ops.prepare_weights(w.astype(np.float32), np.ones(128, np.float32), rank=0)
    with pytest.raises(ValueError):
        ops._ptr(np.zeros((8, 8), np.float32).T)


def test_kernel1_k_limit():
    """smooth_inv is staged in LDS: K above 32768 is refused before any device use."""
    buf, p = _fake(8)
    q = L.lib().svdq_quant_act_lora_down
    assert q(p[0], p[1], p[2], 16, 32768 + 64, 32, 64, 0, p[3], p[4], p[5], None) == L.SVDQ_ERR_UNSUPPORTED_SHAPE
