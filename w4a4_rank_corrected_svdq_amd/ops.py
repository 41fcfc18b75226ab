"""Thin Python binding over the C ABI (argument marshalling only).

Every step of the layer runs in ``libsvdq.so``: host preparation in its C++
code, the forward pass in its two HIP kernels.  PyTorch provides device
memory (``torch.empty``) and the current stream; nothing here computes.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch

from . import _lib as L

__all__ = ["prepare_weights", "quant_act_lora_down", "gemm_w4a4_lora_up", "prepared_bytes",
           "device_check", "lora_down", "lora_up_add", "prepared_bytes_mxfp4", "prepare_weights_mxfp4",
           "quant_act_lora_down_mxfp4", "gemm_mxfp4_lora_up", "gemm_w4a4_lora_up_qkv", "awq_prepare",
           "awq_quant_act", "awq_gemv", "fp6_operand_bytes", "pack_fp6_operand",
           "quant_act_lora_down_fp6", "gemm_w4a4_fp6_lora_up"]


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        if not t.flags.c_contiguous:
            raise ValueError("host arrays passed to the library must be C-contiguous")
        return t.ctypes.data
    return t.data_ptr()


def _dev_arg(name: str, t, dtype, shape, device) -> Optional[int]:
    """Check a device tensor argument (dtype, shape, device, row-major
    contiguity) and return its address."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def device_check(device: int = 0) -> int:
    return L.lib().svdq_device_check(int(device))


def prepared_bytes(K: int, N: int, rank: int, group: int = 64) -> int:
    out = ctypes.c_size_t(0)
    L.check(L.lib().svdq_prepared_bytes(K, N, rank, group, ctypes.byref(out)), "svdq_prepared_bytes")
    return int(out.value)


def _bf16_bits(a) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        if a.dtype != torch.bfloat16:
            raise TypeError("expected a bfloat16 tensor")
        return np.ascontiguousarray(a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError("expected bf16 bit patterns (uint16)")
    return np.ascontiguousarray(a)


def prepare_weights(weight, act_absmax, rank: int = 32, group: int = 64, alpha: float = 0.5,
                    factors=None, power_iters: int = 0, seed: int = 0x5356445175616E74,
                    return_sigma: bool = False) -> dict:
    """Host preparation (svdq_prepare_weights[_ex]).

    weight: [N][K] bf16 (torch tensor or uint16 bits); act_absmax: [K] float32.
    factors: optional (lora_down [r][K], lora_up [N][r]) bf16 bits to use
    instead of the SVD.  Returns numpy arrays: smooth_inv f32 [K], w_codes u8
    [N][K/2], w_scales f16 [K/64][N], lora_down bf16 bits [r][K], lora_up bf16
    bits [N][r] (and sigma [r] f64)."""
    w = _bf16_bits(weight)
    N, K = w.shape
    a = np.ascontiguousarray(np.asarray(act_absmax, dtype=np.float32).reshape(K))
    si = np.empty(K, np.float32)
    wc = np.empty((N, K // 2), np.uint8)
    ws = np.empty((max(K // group, 0), N), np.float16)
    ld = np.empty((rank, K), np.uint16)
    lu = np.empty((N, rank), np.uint16)
    sig = np.empty(max(rank, 1), np.float64)
    fin = (None, None)
    if factors is not None:
        fin = tuple(np.ascontiguousarray(np.asarray(f, dtype=np.uint16)) for f in factors)
        if fin[0].shape != (rank, K) or fin[1].shape != (N, rank):
            raise ValueError("factors must be lora_down [rank][K] and lora_up [N][rank]")
    st = L.lib().svdq_prepare_weights_ex(
        _ptr(w), K, N, _ptr(a), float(alpha), rank, group, _ptr(fin[0]), _ptr(fin[1]),
        int(power_iters), int(seed) & (2 ** 64 - 1), _ptr(si), _ptr(wc), _ptr(ws),
        _ptr(ld) if rank else None, _ptr(lu) if rank else None, _ptr(sig))
    L.check(st, "svdq_prepare_weights")
    out = dict(smooth_inv=si, w_codes=wc, w_scales=ws, lora_down=ld, lora_up=lu,
               rank=rank, group=group, K=K, N=N)
    if return_sigma:
        out["sigma"] = sig[:rank].copy()
    return out


def quant_act_lora_down(x: torch.Tensor, smooth_inv: torch.Tensor, lora_down: Optional[torch.Tensor],
                        rank: int, group: int = 64, act: int = L.SVDQ_ACT_NONE, out=None):
    """Kernel 1 on x's device and current stream.  x: [M][K] bfloat16.
    Returns (x_codes u8 [M][K/2], x_scales f16 [K/64][M], lora_act f32 [M][rank])."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise TypeError("x must be a 2-D bfloat16 CUDA tensor")
    x = x.contiguous()
    M, K = x.shape
    dev = x.device
    if out is None:
        xc = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        xs = torch.empty((K // group, M), dtype=torch.float16, device=dev)
        la = torch.empty((M, rank), dtype=torch.float32, device=dev) if rank else None
    else:
        xc, xs, la = out
    G = K // group if group > 0 else 0
    st = L.lib().svdq_quant_act_lora_down(
        _dev_arg("x", x, torch.bfloat16, (M, K), dev),
        _dev_arg("smooth_inv", smooth_inv, torch.float32, (K,), dev),
        _dev_arg("lora_down", lora_down, torch.bfloat16, (rank, K), dev) if rank else None,
        M, K, rank, group, act,
        _dev_arg("x_codes", xc, torch.uint8, (M, K // 2), dev),
        _dev_arg("x_scales", xs, torch.float16, (G, M), dev),
        _dev_arg("lora_act", la, torch.float32, (M, rank), dev) if rank else None, _stream(dev))
    L.check(st, "svdq_quant_act_lora_down")
    return xc, xs, la


def gemm_w4a4_lora_up(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias,
                      M: int, N: int, K: int, rank: int, group: int = 64,
                      out_dtype: int = L.SVDQ_OUT_BF16, out: Optional[torch.Tensor] = None):
    """Kernel 2 on x_codes' device and current stream; returns y [M][N]."""
    dev = x_codes.device
    if out is None:
        dt = torch.float32 if out_dtype == L.SVDQ_OUT_F32 else torch.bfloat16
        out = torch.empty((M, N), dtype=dt, device=dev)
    G = K // group if group > 0 else 0
    dt = torch.float32 if out_dtype == L.SVDQ_OUT_F32 else torch.bfloat16
    st = L.lib().svdq_gemm_w4a4_lora_up(
        _dev_arg("x_codes", x_codes, torch.uint8, (M, K // 2), dev),
        _dev_arg("x_scales", x_scales, torch.float16, (G, M), dev),
        _dev_arg("w_codes", w_codes, torch.uint8, (N, K // 2), dev),
        _dev_arg("w_scales", w_scales, torch.float16, (G, N), dev),
        _dev_arg("lora_act", lora_act, torch.float32, (M, rank), dev) if rank else None,
        _dev_arg("lora_up", lora_up, torch.bfloat16, (N, rank), dev) if rank else None,
        _dev_arg("bias", bias, torch.bfloat16, (N,), dev),
        M, N, K, rank, group, out_dtype, _dev_arg("y", out, dt, (M, N), dev), _stream(dev))
    L.check(st, "svdq_gemm_w4a4_lora_up")
    return out


# ------------------------------------------------- INT4 codes on the 6-bit MFMA
def fp6_operand_bytes(rows: int, K: int, layout: int) -> int:
    out = ctypes.c_size_t(0)
    L.check(L.lib().svdq_fp6_operand_bytes(rows, K, layout, ctypes.byref(out)), "svdq_fp6_operand_bytes")
    return int(out.value)


def pack_fp6_operand(codes, layout: int = L.SVDQ_FP6_WEIGHTS) -> np.ndarray:
    """Host re-pack of nibble codes [rows][K/2] u8 into the fragment layout
    (svdq_pack_fp6_operand); returns u8 [K/64][RB][1536]."""
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    rows, K = c.shape[0], 2 * c.shape[1]
    nbytes = fp6_operand_bytes(rows, K, layout)
    out = np.empty(nbytes, np.uint8)
    L.check(L.lib().svdq_pack_fp6_operand(_ptr(c), rows, K, layout, _ptr(out)), "svdq_pack_fp6_operand")
    return out.reshape(K // 64, -1, 1536)


def quant_act_lora_down_fp6(x: torch.Tensor, smooth_inv: torch.Tensor, lora_down: Optional[torch.Tensor],
                            rank: int, group: int = 64, act: int = L.SVDQ_ACT_NONE, out=None):
    """Kernel 1 with the codes in the 6-bit fragment layout.  Returns
    (x_fp6 u8 [K/64][ceil(M/32)][1536], x_scales f16 [K/64][Mp], lora_act
    f32 [M][rank]), Mp = 32 ceil(M/32)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise TypeError("x must be a 2-D bfloat16 CUDA tensor")
    x = x.contiguous()
    M, K = x.shape
    dev = x.device
    G = K // group if group > 0 else 0
    RB = (M + 31) // 32
    if out is None:
        xf = torch.empty((G, RB, 1536), dtype=torch.uint8, device=dev)
        xs = torch.empty((G, 32 * RB), dtype=torch.float16, device=dev)
        la = torch.empty((M, rank), dtype=torch.float32, device=dev) if rank else None
    else:
        xf, xs, la = out
    st = L.lib().svdq_quant_act_lora_down_fp6(
        _dev_arg("x", x, torch.bfloat16, (M, K), dev),
        _dev_arg("smooth_inv", smooth_inv, torch.float32, (K,), dev),
        _dev_arg("lora_down", lora_down, torch.bfloat16, (rank, K), dev) if rank else None,
        M, K, rank, group, act,
        _dev_arg("x_fp6", xf, torch.uint8, (G, RB, 1536), dev),
        _dev_arg("x_scales", xs, torch.float16, (G, 32 * RB), dev),
        _dev_arg("lora_act", la, torch.float32, (M, rank), dev) if rank else None, _stream(dev))
    L.check(st, "svdq_quant_act_lora_down_fp6")
    return xf, xs, la


def gemm_w4a4_fp6_lora_up(x_fp6, x_scales, w_fp6, w_scales, lora_act, lora_up, bias,
                          M: int, N: int, K: int, rank: int, group: int = 64,
                          out_dtype: int = L.SVDQ_OUT_BF16, out: Optional[torch.Tensor] = None):
    """Kernel 2 on the 6-bit MFMA; returns y [M][N]."""
    dev = x_fp6.device
    dt = torch.float32 if out_dtype == L.SVDQ_OUT_F32 else torch.bfloat16
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=dev)
    G = K // group if group > 0 else 0
    RBa, RBb = (M + 31) // 32, 4 * ((N + 127) // 128)
    st = L.lib().svdq_gemm_w4a4_fp6_lora_up(
        _dev_arg("x_fp6", x_fp6, torch.uint8, (G, RBa, 1536), dev),
        _dev_arg("x_scales", x_scales, torch.float16, (G, 32 * RBa), dev),
        _dev_arg("w_fp6", w_fp6, torch.uint8, (G, RBb, 1536), dev),
        _dev_arg("w_scales", w_scales, torch.float16, (G, N), dev),
        _dev_arg("lora_act", lora_act, torch.float32, (M, rank), dev) if rank else None,
        _dev_arg("lora_up", lora_up, torch.bfloat16, (N, rank), dev) if rank else None,
        _dev_arg("bias", bias, torch.bfloat16, (N,), dev),
        M, N, K, rank, group, out_dtype, _dev_arg("y", out, dt, (M, N), dev), _stream(dev))
    L.check(st, "svdq_gemm_w4a4_fp6_lora_up")
    return out


def gemm_w4a4_fp6_lora_up_n192(x_fp6, x_scales, w_fp6_rows, w_scales, lora_act, lora_up, bias,
                               M: int, N: int, K: int, rank: int, group: int = 64,
                               out_dtype: int = L.SVDQ_OUT_BF16, out: Optional[torch.Tensor] = None):
    """Kernel 2 on the 6-bit MFMA in 256 x 192 tiles (weights in the plain
    fragment layout, N % 192 == 0); returns y [M][N]."""
    dev = x_fp6.device
    dt = torch.float32 if out_dtype == L.SVDQ_OUT_F32 else torch.bfloat16
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=dev)
    G = K // group if group > 0 else 0
    RBa, RBw = (M + 31) // 32, (N + 31) // 32
    st = L.lib().svdq_gemm_w4a4_fp6_lora_up_n192(
        _dev_arg("x_fp6", x_fp6, torch.uint8, (G, RBa, 1536), dev),
        _dev_arg("x_scales", x_scales, torch.float16, (G, 32 * RBa), dev),
        _dev_arg("w_fp6_rows", w_fp6_rows, torch.uint8, (G, RBw, 1536), dev),
        _dev_arg("w_scales", w_scales, torch.float16, (G, N), dev),
        _dev_arg("lora_act", lora_act, torch.float32, (M, rank), dev) if rank else None,
        _dev_arg("lora_up", lora_up, torch.bfloat16, (N, rank), dev) if rank else None,
        _dev_arg("bias", bias, torch.bfloat16, (N,), dev),
        M, N, K, rank, group, out_dtype, _dev_arg("y", out, dt, (M, N), dev), _stream(dev))
    L.check(st, "svdq_gemm_w4a4_fp6_lora_up_n192")
    return out


def fp6_n192_preferred(M: int, N: int) -> bool:
    """Whether the 256 x 192 form of the 6-bit kernel 2 is expected to be the
    faster one for an M x N output on the current device."""
    return bool(L.lib().svdq_fp6_n192_preferred(int(M), int(N)))


def int4_route(M: int, N: int) -> int:
    """The kernels expected to be fastest for an INT4 layer's M x N output on
    the current device: 0 6-bit kernel 2 in 256 x 256 tiles, 1 in 256 x 192
    tiles, 2 the int8 engine (svdq_int4_route)."""
    return int(L.lib().svdq_int4_route(int(M), int(N)))


def gemm_w4a4_fp6_lora_up_qkv(x_fp6, x_scales, w_fp6, w_scales, lora_act, lora_up, bias, norm_q, norm_k,
                              rope_cos, rope_sin, M: int, N: int, K: int, rank: int, eps: float = 1e-6,
                              group: int = 64, out_dtype: int = L.SVDQ_OUT_BF16,
                              out: Optional[torch.Tensor] = None):
    """Kernel 2 on the 6-bit MFMA with the fused QKV epilogue (per-head Q/K
    RMSNorm + rotary embedding); returns y [M][N] with N = 3 * heads * 128."""
    dev = x_fp6.device
    dt = torch.float32 if out_dtype == L.SVDQ_OUT_F32 else torch.bfloat16
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=dev)
    G = K // group if group > 0 else 0
    RBa, RBb = (M + 31) // 32, 4 * ((N + 127) // 128)
    st = L.lib().svdq_gemm_w4a4_fp6_lora_up_qkv(
        _dev_arg("x_fp6", x_fp6, torch.uint8, (G, RBa, 1536), dev),
        _dev_arg("x_scales", x_scales, torch.float16, (G, 32 * RBa), dev),
        _dev_arg("w_fp6", w_fp6, torch.uint8, (G, RBb, 1536), dev),
        _dev_arg("w_scales", w_scales, torch.float16, (G, N), dev),
        _dev_arg("lora_act", lora_act, torch.float32, (M, rank), dev) if rank else None,
        _dev_arg("lora_up", lora_up, torch.bfloat16, (N, rank), dev) if rank else None,
        _dev_arg("bias", bias, torch.bfloat16, (N,), dev),
        _dev_arg("norm_q", norm_q, torch.bfloat16, (128,), dev),
        _dev_arg("norm_k", norm_k, torch.bfloat16, (128,), dev),
        _dev_arg("rope_cos", rope_cos, torch.float32, (M, 64), dev),
        _dev_arg("rope_sin", rope_sin, torch.float32, (M, 64), dev),
        float(eps), M, N, K, rank, group, out_dtype, _dev_arg("y", out, dt, (M, N), dev), _stream(dev))
    L.check(st, "svdq_gemm_w4a4_fp6_lora_up_qkv")
    return out


def mlp_chain_workspace_bytes(M: int, N: int, rank_dn: int) -> int:
    out = ctypes.c_size_t(0)
    L.check(L.lib().svdq_mlp_chain_workspace_bytes(M, N, rank_dn, ctypes.byref(out)), "svdq_mlp_chain_workspace_bytes")
    return int(out.value)


def gemm_w4a4_fp6_mlp_chain(x_fp6, x_scales, w_fp6, w_scales, lora_act, lora_up, bias, M: int, N: int, K: int,
                            rank: int, smooth_inv_dn, lora_down_dn, rank_dn: int, group: int = 64,
                            out=None, workspace: Optional[torch.Tensor] = None):
    """The up layer's kernel 2 with the down layer's kernel 1 in its epilogue
    (svdq_gemm_w4a4_fp6_mlp_chain).  Returns the down layer's (x_fp6
    [N/64][ceil(M/32)][1536] u8, x_scales [N/64][Mp] f16, lora_act [M][rank_dn]
    f32)."""
    dev = x_fp6.device
    G, Gd, RB = K // group, N // 64, (M + 31) // 32
    if out is None:
        xf = torch.empty((Gd, RB, 1536), dtype=torch.uint8, device=dev)
        xs = torch.empty((Gd, 32 * RB), dtype=torch.float16, device=dev)
        la = torch.empty((M, rank_dn), dtype=torch.float32, device=dev) if rank_dn else None
    else:
        xf, xs, la = out
    need = mlp_chain_workspace_bytes(M, N, rank_dn)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    RBb = 4 * ((N + 127) // 128)
    st = L.lib().svdq_gemm_w4a4_fp6_mlp_chain(
        _dev_arg("x_fp6", x_fp6, torch.uint8, (G, RB, 1536), dev),
        _dev_arg("x_scales", x_scales, torch.float16, (G, 32 * RB), dev),
        _dev_arg("w_fp6", w_fp6, torch.uint8, (G, RBb, 1536), dev),
        _dev_arg("w_scales", w_scales, torch.float16, (G, N), dev),
        _dev_arg("lora_act", lora_act, torch.float32, (M, rank), dev) if rank else None,
        _dev_arg("lora_up", lora_up, torch.bfloat16, (N, rank), dev) if rank else None,
        _dev_arg("bias", bias, torch.bfloat16, (N,), dev),
        M, N, K, rank, group,
        _dev_arg("smooth_inv_dn", smooth_inv_dn, torch.float32, (N,), dev),
        _dev_arg("lora_down_dn", lora_down_dn, torch.bfloat16, (rank_dn, N), dev) if rank_dn else None, rank_dn,
        _dev_arg("x_fp6_dn", xf, torch.uint8, (Gd, RB, 1536), dev),
        _dev_arg("x_scales_dn", xs, torch.float16, (Gd, 32 * RB), dev),
        _dev_arg("lora_act_dn", la, torch.float32, (M, rank_dn), dev) if rank_dn else None,
        _ptr(workspace) if need else None, int(workspace.numel()) if (need and workspace is not None) else 0,
        _stream(dev))
    L.check(st, "svdq_gemm_w4a4_fp6_mlp_chain")
    return xf, xs, la


def lora_down(x: torch.Tensor, smooth_inv: torch.Tensor, lora_down_w: torch.Tensor, rank: int,
              group: int = 64, act: int = L.SVDQ_ACT_NONE, out: Optional[torch.Tensor] = None):
    """Unfused down projection (reads x again): lora_act [M][rank] fp32."""
    x = x.contiguous()
    M, K = x.shape
    dev = x.device
    if out is None:
        out = torch.empty((M, rank), dtype=torch.float32, device=dev)
    st = L.lib().svdq_lora_down(
        _dev_arg("x", x, torch.bfloat16, (M, K), dev),
        _dev_arg("smooth_inv", smooth_inv, torch.float32, (K,), dev),
        _dev_arg("lora_down", lora_down_w, torch.bfloat16, (rank, K), dev),
        M, K, rank, group, act, _dev_arg("lora_act", out, torch.float32, (M, rank), dev), _stream(dev))
    L.check(st, "svdq_lora_down")
    return out


def lora_up_add(lora_act: torch.Tensor, lora_up_w: torch.Tensor, y: torch.Tensor):
    """Unfused up projection: y = bf16(y + bf16(lora_act) lora_up^T), in place."""
    M, rank = lora_act.shape
    N = y.shape[1]
    dev = y.device
    st = L.lib().svdq_lora_up_add(
        _dev_arg("lora_act", lora_act, torch.float32, (M, rank), dev),
        _dev_arg("lora_up", lora_up_w, torch.bfloat16, (N, rank), dev),
        M, N, rank, _dev_arg("y", y, torch.bfloat16, (M, N), dev), _stream(dev))
    L.check(st, "svdq_lora_up_add")
    return y


# ---------------------------------------------------------------- MXFP4 variant
def prepared_bytes_mxfp4(K: int, N: int, rank: int) -> int:
    out = ctypes.c_size_t(0)
    L.check(L.lib().svdq_prepared_bytes_mxfp4(K, N, rank, ctypes.byref(out)), "svdq_prepared_bytes_mxfp4")
    return int(out.value)


def prepare_weights_mxfp4(weight, act_absmax, rank: int = 32, alpha: float = 0.5, factors=None,
                          power_iters: int = 0, seed: int = 0x5356445175616E74,
                          return_sigma: bool = False) -> dict:
    """Host preparation with the MXFP4 residual (svdq_prepare_weights_mxfp4).
    Returns numpy arrays: smooth_inv f32 [K], w_codes u8 [N][K/2] (E2M1),
    w_scales u8 [N][K/32] (E8M0), lora_down / lora_up bf16 bits."""
    w = _bf16_bits(weight)
    N, K = w.shape
    a = np.ascontiguousarray(np.asarray(act_absmax, dtype=np.float32).reshape(K))
    si = np.empty(K, np.float32)
    wc = np.empty((N, K // 2), np.uint8)
    ws = np.empty((N, max(K // 32, 0)), np.uint8)
    ld = np.empty((rank, K), np.uint16)
    lu = np.empty((N, rank), np.uint16)
    sig = np.empty(max(rank, 1), np.float64)
    fin = (None, None)
    if factors is not None:
        fin = tuple(np.ascontiguousarray(np.asarray(f, dtype=np.uint16)) for f in factors)
        if fin[0].shape != (rank, K) or fin[1].shape != (N, rank):
            raise ValueError("factors must be lora_down [rank][K] and lora_up [N][rank]")
    st = L.lib().svdq_prepare_weights_mxfp4(
        _ptr(w), K, N, _ptr(a), float(alpha), rank, _ptr(fin[0]), _ptr(fin[1]),
        int(power_iters), int(seed) & (2 ** 64 - 1), _ptr(si), _ptr(wc), _ptr(ws),
        _ptr(ld) if rank else None, _ptr(lu) if rank else None, _ptr(sig))
    L.check(st, "svdq_prepare_weights_mxfp4")
    out = dict(smooth_inv=si, w_codes=wc, w_scales=ws, lora_down=ld, lora_up=lu,
               rank=rank, group=32, K=K, N=N, precision="mxfp4")
    if return_sigma:
        out["sigma"] = sig[:rank].copy()
    return out


def quant_act_lora_down_mxfp4(x: torch.Tensor, smooth_inv: torch.Tensor, lora_down: Optional[torch.Tensor],
                              rank: int, act: int = L.SVDQ_ACT_NONE, out=None):
    """Kernel 1 with the MXFP4 quantizer.  Returns (x_codes u8 [M][K/2],
    x_scales u8 [M][K/32], lora_act f32 [M][rank])."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise TypeError("x must be a 2-D bfloat16 CUDA tensor")
    x = x.contiguous()
    M, K = x.shape
    dev = x.device
    if out is None:
        xc = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        xs = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
        la = torch.empty((M, rank), dtype=torch.float32, device=dev) if rank else None
    else:
        xc, xs, la = out
    st = L.lib().svdq_quant_act_lora_down_mxfp4(
        _dev_arg("x", x, torch.bfloat16, (M, K), dev),
        _dev_arg("smooth_inv", smooth_inv, torch.float32, (K,), dev),
        _dev_arg("lora_down", lora_down, torch.bfloat16, (rank, K), dev) if rank else None,
        M, K, rank, act,
        _dev_arg("x_codes", xc, torch.uint8, (M, K // 2), dev),
        _dev_arg("x_scales", xs, torch.uint8, (M, K // 32), dev),
        _dev_arg("lora_act", la, torch.float32, (M, rank), dev) if rank else None, _stream(dev))
    L.check(st, "svdq_quant_act_lora_down_mxfp4")
    return xc, xs, la


def gemm_mxfp4_lora_up(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias,
                       M: int, N: int, K: int, rank: int, out_dtype: int = L.SVDQ_OUT_BF16,
                       out: Optional[torch.Tensor] = None):
    """Kernel 2 for MXFP4 operands; returns y [M][N]."""
    dev = x_codes.device
    dt = torch.float32 if out_dtype == L.SVDQ_OUT_F32 else torch.bfloat16
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=dev)
    st = L.lib().svdq_gemm_mxfp4_lora_up(
        _dev_arg("x_codes", x_codes, torch.uint8, (M, K // 2), dev),
        _dev_arg("x_scales", x_scales, torch.uint8, (M, K // 32), dev),
        _dev_arg("w_codes", w_codes, torch.uint8, (N, K // 2), dev),
        _dev_arg("w_scales", w_scales, torch.uint8, (N, K // 32), dev),
        _dev_arg("lora_act", lora_act, torch.float32, (M, rank), dev) if rank else None,
        _dev_arg("lora_up", lora_up, torch.bfloat16, (N, rank), dev) if rank else None,
        _dev_arg("bias", bias, torch.bfloat16, (N,), dev),
        M, N, K, rank, out_dtype, _dev_arg("y", out, dt, (M, N), dev), _stream(dev))
    L.check(st, "svdq_gemm_mxfp4_lora_up")
    return out


def gemm_w4a4_lora_up_qkv(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, norm_q, norm_k,
                          rope_cos, rope_sin, M: int, N: int, K: int, rank: int, eps: float = 1e-6,
                          group: int = 64, out_dtype: int = L.SVDQ_OUT_BF16, out: Optional[torch.Tensor] = None):
    """Kernel 2 with the fused QKV epilogue (per-head Q/K RMSNorm + rotary
    embedding); returns y [M][N] with N = 3 * heads * 128."""
    dev = x_codes.device
    dt = torch.float32 if out_dtype == L.SVDQ_OUT_F32 else torch.bfloat16
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=dev)
    G = K // group if group > 0 else 0
    st = L.lib().svdq_gemm_w4a4_lora_up_qkv(
        _dev_arg("x_codes", x_codes, torch.uint8, (M, K // 2), dev),
        _dev_arg("x_scales", x_scales, torch.float16, (G, M), dev),
        _dev_arg("w_codes", w_codes, torch.uint8, (N, K // 2), dev),
        _dev_arg("w_scales", w_scales, torch.float16, (G, N), dev),
        _dev_arg("lora_act", lora_act, torch.float32, (M, rank), dev) if rank else None,
        _dev_arg("lora_up", lora_up, torch.bfloat16, (N, rank), dev) if rank else None,
        _dev_arg("bias", bias, torch.bfloat16, (N,), dev),
        _dev_arg("norm_q", norm_q, torch.bfloat16, (128,), dev),
        _dev_arg("norm_k", norm_k, torch.bfloat16, (128,), dev),
        _dev_arg("rope_cos", rope_cos, torch.float32, (M, 64), dev),
        _dev_arg("rope_sin", rope_sin, torch.float32, (M, 64), dev),
        float(eps), M, N, K, rank, group, out_dtype, _dev_arg("y", out, dt, (M, N), dev), _stream(dev))
    L.check(st, "svdq_gemm_w4a4_lora_up_qkv")
    return out


# ---------------------------------------------------------------- AWQ W4A16
def awq_prepare(weight, x_cal, alpha: float = -1.0, group: int = 64) -> dict:
    """Host AWQ preparation (svdq_awq_prepare).  weight [N][K] and x_cal
    [Mc][K] bf16 (tensors or uint16 bits); alpha < 0 searches the grid.
    Returns numpy arrays: inv_scale f32 [K], w_codes u8 [N][K/2], w_scales
    f16 [N][K/64], w_zeros u8 [N][K/64], and alpha."""
    w = _bf16_bits(weight)
    xc = _bf16_bits(x_cal)
    N, K = w.shape
    Mc = xc.shape[0]
    if xc.shape[1] != K:
        raise ValueError("x_cal must be [Mc][K]")
    inv = np.empty(K, np.float32)
    wc = np.empty((N, K // 2), np.uint8)
    ws = np.empty((N, max(K // group, 0)), np.float16)
    wz = np.empty((N, max(K // group, 0)), np.uint8)
    al = ctypes.c_double(0.0)
    st = L.lib().svdq_awq_prepare(_ptr(w), K, N, _ptr(xc), Mc, float(alpha), group, _ptr(inv), _ptr(wc),
                                  _ptr(ws), _ptr(wz), ctypes.addressof(al))
    L.check(st, "svdq_awq_prepare")
    return dict(inv_scale=inv, w_codes=wc, w_scales=ws, w_zeros=wz, alpha=float(al.value), K=K, N=N, group=group)


def awq_quant_act(x: torch.Tensor, inv_scale: torch.Tensor, out=None):
    """x_hat [M][K] bf16 and xsum [K/64][16] fp32 (svdq_awq_quant_act)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise TypeError("x must be a 2-D bfloat16 CUDA tensor")
    x = x.contiguous()
    M, K = x.shape
    dev = x.device
    if out is None:
        xh = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        xs = torch.empty((K // 64, 16), dtype=torch.float32, device=dev)
    else:
        xh, xs = out
    st = L.lib().svdq_awq_quant_act(_dev_arg("x", x, torch.bfloat16, (M, K), dev),
                                    _dev_arg("inv_scale", inv_scale, torch.float32, (K,), dev), M, K,
                                    _dev_arg("x_hat", xh, torch.bfloat16, (M, K), dev),
                                    _dev_arg("xsum", xs, torch.float32, (K // 64, 16), dev), _stream(dev))
    L.check(st, "svdq_awq_quant_act")
    return xh, xs


def awq_gemv(x_hat, xsum, w_codes, w_scales, w_zeros, bias, M: int, N: int, K: int,
             out: Optional[torch.Tensor] = None):
    """y [M][N] bf16 (svdq_awq_gemv)."""
    dev = x_hat.device
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    G = K // 64
    st = L.lib().svdq_awq_gemv(
        _dev_arg("x_hat", x_hat, torch.bfloat16, (M, K), dev),
        _dev_arg("xsum", xsum, torch.float32, (G, 16), dev),
        _dev_arg("w_codes", w_codes, torch.uint8, (N, K // 2), dev),
        _dev_arg("w_scales", w_scales, torch.float16, (N, G), dev),
        _dev_arg("w_zeros", w_zeros, torch.uint8, (N, G), dev),
        _dev_arg("bias", bias, torch.bfloat16, (N,), dev),
        M, N, K, _dev_arg("y", out, torch.bfloat16, (M, N), dev), _stream(dev))
    L.check(st, "svdq_awq_gemv")
    return out


def awq_linear_row(x, inv_scale, w_codes, w_scales, w_zeros, bias, N: int, K: int,
                   out: Optional[torch.Tensor] = None):
    """y [1][N] bf16 from one row x [1][K] (svdq_awq_linear_row: the
    activation scaling and the GEMV in one launch, bit for bit their output)."""
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.numel() != K:
        raise TypeError("x must be one bfloat16 CUDA row of K values")
    x = x.contiguous().view(1, K)
    dev = x.device
    if out is None:
        out = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
    G = K // 64
    st = L.lib().svdq_awq_linear_row(
        _dev_arg("x", x, torch.bfloat16, (1, K), dev),
        _dev_arg("inv_scale", inv_scale, torch.float32, (K,), dev),
        _dev_arg("w_codes", w_codes, torch.uint8, (N, K // 2), dev),
        _dev_arg("w_scales", w_scales, torch.float16, (N, G), dev),
        _dev_arg("w_zeros", w_zeros, torch.uint8, (N, G), dev),
        _dev_arg("bias", bias, torch.bfloat16, (N,), dev),
        N, K, _dev_arg("y", out, torch.bfloat16, (1, N), dev), _stream(dev))
    L.check(st, "svdq_awq_linear_row")
    return out
