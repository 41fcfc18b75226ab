"""``SVDQW4A4Linear``: a prepared layer resident in device memory.

Mirrors the pages' module-level interface (``SVDQW4A4Linear.from_linear``,
"Quantizing models with structural rewrites" in "Bringing Nunchaku 4-bit
Diffusion Inference to Diffusers"; precision / group_size / rank fields of the
``quantization_config`` in "Native loading in Diffusers").  Preparation runs
in the library's host code, the forward pass in its two HIP kernels.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import _lib as L
from . import ops


def _bits_to_bf16(bits: np.ndarray, device) -> torch.Tensor:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(device)


def _to_dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class SVDQW4A4Linear:
    """One prepared layer.  ``precision`` is "int4" (group 64, fp16 scales)
    or "mxfp4" (E2M1 codes, E8M0 scale per 32), as in the prepared dict.

    An int4 layer runs on one of two engines: "fp6" (default) feeds the INT4
    codes to the 6-bit float MFMA in their E3M2 containers
    (``svdq_quant_act_lora_down_fp6`` + ``svdq_gemm_w4a4_fp6_lora_up``;
    the weights are re-packed once here), "int8" to the int8 MFMA from the
    nibble layout (``svdq_quant_act_lora_down`` +
    ``svdq_gemm_w4a4_lora_up``).  Both compute the same layer; the nibble
    codes stay resident for the int8 engine, the unfused comparison path and
    the fused QKV epilogue.  With N % 192 == 0 the 6-bit engine also keeps
    the weights in the plain row-block layout for its 256 x 192 tile form
    (``svdq_gemm_w4a4_fp6_lora_up_n192``), used per call where
    ``svdq_fp6_n192_preferred`` says so; ``n192=False`` drops that copy.
    For few rows (256-row tiles covering fewer than half the CUs) forward()
    of a 6-bit layer runs the int8 engine's kernels, whose 128 x 128 form
    keeps more CUs busy (``route``); ``auto_route=False`` keeps it on the
    6-bit kernels."""

    def __init__(self, prepared: dict, bias: Optional[torch.Tensor], device, engine: str = "fp6",
                 n192: bool = True, auto_route: bool = True):
        dev = torch.device(device)
        self.precision = prepared.get("precision", "int4")
        if self.precision not in ("int4", "mxfp4"):
            raise ValueError(f"unknown precision {self.precision!r}")
        if engine not in ("fp6", "int8"):
            raise ValueError(f"unknown engine {engine!r}")
        self.engine = engine if self.precision == "int4" else "mxfp4"
        self.K, self.N = prepared["K"], prepared["N"]
        self.rank, self.group = prepared["rank"], prepared["group"]
        self.smooth_inv = _to_dev(np.asarray(prepared["smooth_inv"], np.float32), dev)
        self.w_codes = _to_dev(np.asarray(prepared["w_codes"], np.uint8), dev)
        sdt = np.uint8 if self.precision == "mxfp4" else np.float16
        self.w_scales = _to_dev(np.asarray(prepared["w_scales"], sdt), dev)
        self.lora_down = _bits_to_bf16(prepared["lora_down"], dev) if self.rank else None
        self.lora_up = _bits_to_bf16(prepared["lora_up"], dev) if self.rank else None
        self.bias = None if bias is None else bias.detach().to(dev, torch.bfloat16).contiguous()
        self.w_fp6 = None
        self.w_fp6_rows = None
        self._n192_choice = {}
        self._route_choice = {}
        self.auto_route = auto_route
        if self.engine == "fp6":
            codes = np.asarray(prepared["w_codes"], np.uint8).reshape(self.N, self.K // 2)
            self.w_fp6 = _to_dev(ops.pack_fp6_operand(codes, L.SVDQ_FP6_WEIGHTS), dev)
            if n192 and self.N % 192 == 0:
                # the plain row-block copy for the 256 x 192 tile form, taken
                # where it fills the CUs in fewer rounds (svdq_fp6_n192_preferred);
                # a second 6-bit weight copy (0.75 K N bytes): n192=False
                # leaves it out and always runs the 256 x 256 form
                self.w_fp6_rows = _to_dev(ops.pack_fp6_operand(codes, L.SVDQ_FP6_ACTIVATIONS), dev)

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, act_absmax, rank: int = 32, group: int = 64,
                    alpha: float = 0.5, device="cuda", precision: str = "int4", engine: str = "fp6",
                    n192: bool = True, auto_route: bool = True):
        """Quantize a ``torch.nn.Linear`` (weight [out][in], bf16) given the
        calibration statistic ``act_absmax`` [in] (max |x| per input channel)."""
        w = linear.weight.detach().to(torch.bfloat16).cpu()
        a = np.asarray(act_absmax, np.float32)
        if precision == "mxfp4":
            prep = ops.prepare_weights_mxfp4(w, a, rank, alpha)
        elif precision == "int4":
            prep = ops.prepare_weights(w, a, rank, group, alpha)
        else:
            raise ValueError(f"unknown precision {precision!r}")
        return cls(prep, linear.bias, device, engine, n192, auto_route)

    def route(self, M: int) -> str:
        """The engine whose kernels forward() runs for M rows: the layer's
        own, except that an "fp6" layer with auto_route takes the int8
        engine's kernels where its 256-row tiles would cover fewer than half
        the CUs (svdq_int4_route; the nibble codes are resident anyway)."""
        if self.engine != "fp6" or not self.auto_route:
            return self.engine
        hit = self._route_choice.get(M)
        if hit is None:
            hit = self._route_choice[M] = "int8" if ops.int4_route(M, self.N) == 2 else "fp6"
        return hit

    def forward(self, x: torch.Tensor, act: int = L.SVDQ_ACT_NONE, out_dtype: int = L.SVDQ_OUT_BF16):
        M = x.shape[0]
        if self.route(M) == "fp6":
            xf, xs, la = ops.quant_act_lora_down_fp6(x, self.smooth_inv, self.lora_down, self.rank, self.group, act)
            return self.kernel2_fp6(xf, xs, la, M, out_dtype)
        if self.precision == "mxfp4":
            xc, xs, la = ops.quant_act_lora_down_mxfp4(x, self.smooth_inv, self.lora_down, self.rank, act)
            return ops.gemm_mxfp4_lora_up(xc, xs, self.w_codes, self.w_scales, la, self.lora_up, self.bias,
                                          M, self.N, self.K, self.rank, out_dtype)
        xc, xs, la = ops.quant_act_lora_down(x, self.smooth_inv, self.lora_down, self.rank, self.group, act)
        return ops.gemm_w4a4_lora_up(xc, xs, self.w_codes, self.w_scales, la, self.lora_up, self.bias,
                                     M, self.N, self.K, self.rank, self.group, out_dtype)

    __call__ = forward

    def _n192(self, M: int) -> bool:
        # the tile-form choice per row count, asked of the library once
        hit = self._n192_choice.get(M)
        if hit is None:
            hit = self._n192_choice[M] = ops.fp6_n192_preferred(M, self.N)
        return hit

    def kernel2_fp6(self, x_fp6, x_scales, lora_act, M: int, out_dtype: int = L.SVDQ_OUT_BF16,
                    out: Optional[torch.Tensor] = None):
        """Kernel 2 of the 6-bit engine on kernel 1's outputs: the 256 x 192
        tile form where it fills the CUs in fewer rounds, else 256 x 256."""
        if self.w_fp6_rows is not None and self._n192(M):
            return ops.gemm_w4a4_fp6_lora_up_n192(x_fp6, x_scales, self.w_fp6_rows, self.w_scales, lora_act,
                                                  self.lora_up, self.bias, M, self.N, self.K, self.rank, self.group,
                                                  out_dtype, out=out)
        return ops.gemm_w4a4_fp6_lora_up(x_fp6, x_scales, self.w_fp6, self.w_scales, lora_act, self.lora_up,
                                         self.bias, M, self.N, self.K, self.rank, self.group, out_dtype, out=out)

    def forward_qkv(self, x: torch.Tensor, norm_q: torch.Tensor, norm_k: torch.Tensor,
                    rope_cos: Optional[torch.Tensor] = None, rope_sin: Optional[torch.Tensor] = None,
                    eps: float = 1e-6, out_dtype: int = L.SVDQ_OUT_BF16):
        """The fused QKV operator of a layer whose weight is [W_q; W_k; W_v]
        (N = 3 heads 128): the projection, then per-head RMSNorm of the Q and
        K heads (bf16 weights norm_q, norm_k [128]) and, given rope_cos /
        rope_sin [M][64] fp32, the rotary embedding of their adjacent pairs;
        V as projected.  INT4 layers only (either engine)."""
        M = x.shape[0]
        if self.engine == "fp6":
            xf, xs, la = ops.quant_act_lora_down_fp6(x, self.smooth_inv, self.lora_down, self.rank, self.group)
            return ops.gemm_w4a4_fp6_lora_up_qkv(xf, xs, self.w_fp6, self.w_scales, la, self.lora_up, self.bias,
                                                 norm_q, norm_k, rope_cos, rope_sin, M, self.N, self.K, self.rank,
                                                 eps, self.group, out_dtype)
        if self.precision != "int4":
            raise ValueError("the fused QKV epilogue runs on INT4 layers")
        xc, xs, la = ops.quant_act_lora_down(x, self.smooth_inv, self.lora_down, self.rank, self.group)
        return ops.gemm_w4a4_lora_up_qkv(xc, xs, self.w_codes, self.w_scales, la, self.lora_up, self.bias,
                                         norm_q, norm_k, rope_cos, rope_sin, M, self.N, self.K, self.rank,
                                         eps, self.group, out_dtype)


class SVDQMLPChain:
    """An MLP pair (up layer, tanh-GELU, down layer), both on the 6-bit
    engine, run as a chain: kernel 1 of the up layer, the up layer's kernel 2
    with the down layer's kernel 1 in its epilogue (the up output never goes
    to memory), then the down layer's kernel 2.  The result is the 6-bit
    two-layer path's ``down(up(x), act=GELU)`` (modules with auto_route off)
    up to the fp32 rounding of the down projection's per-slice partials."""

    def __init__(self, up: SVDQW4A4Linear, down: SVDQW4A4Linear):
        if up.engine != "fp6" or down.engine != "fp6":
            raise ValueError("the chain runs both layers on the 6-bit engine")
        if down.K != up.N:
            raise ValueError(f"the down layer's K ({down.K}) is not the up layer's N ({up.N})")
        self.up, self.down = up, down
        self._ws = None

    def forward(self, x: torch.Tensor, out_dtype: int = L.SVDQ_OUT_BF16):
        up, dn = self.up, self.down
        M = x.shape[0]
        xf, xs, la = ops.quant_act_lora_down_fp6(x, up.smooth_inv, up.lora_down, up.rank, up.group)
        need = ops.mlp_chain_workspace_bytes(M, up.N, dn.rank)
        if need and (self._ws is None or self._ws.numel() < need or self._ws.device != x.device):
            self._ws = torch.empty(need, dtype=torch.uint8, device=x.device)
        xf2, xs2, la2 = ops.gemm_w4a4_fp6_mlp_chain(xf, xs, up.w_fp6, up.w_scales, la, up.lora_up, up.bias,
                                                    M, up.N, up.K, up.rank, dn.smooth_inv, dn.lora_down, dn.rank,
                                                    up.group, workspace=self._ws if need else None)
        return dn.kernel2_fp6(xf2, xs2, la2, M, out_dtype)

    __call__ = forward


class AWQW4A16Linear:
    """AWQ W4A16 layer (the pages' runtime layer name for the modulation
    projections): 4-bit weights with activation-aware channel scales, bf16
    activations, a few rows per call."""

    def __init__(self, prepared: dict, bias: Optional[torch.Tensor], device):
        dev = torch.device(device)
        self.K, self.N, self.group = prepared["K"], prepared["N"], prepared["group"]
        self.alpha = prepared.get("alpha")
        self.inv_scale = _to_dev(np.asarray(prepared["inv_scale"], np.float32), dev)
        self.w_codes = _to_dev(np.asarray(prepared["w_codes"], np.uint8), dev)
        self.w_scales = _to_dev(np.asarray(prepared["w_scales"], np.float16), dev)
        self.w_zeros = _to_dev(np.asarray(prepared["w_zeros"], np.uint8), dev)
        self.bias = None if bias is None else bias.detach().to(dev, torch.bfloat16).contiguous()

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, x_cal, alpha: float = -1.0, device="cuda"):
        """Quantize a ``torch.nn.Linear`` given calibration activations
        ``x_cal`` [Mc][in] (bf16); alpha < 0 searches the grid."""
        w = linear.weight.detach().to(torch.bfloat16).cpu()
        xc = torch.as_tensor(x_cal).to(torch.bfloat16).cpu()
        return cls(ops.awq_prepare(w, xc, alpha), linear.bias, device)

    def forward(self, x: torch.Tensor):
        M = x.shape[0]
        if M == 1 and self.K <= L.SVDQ_AWQ_ROW_MAX_K:
            # one conditioning vector: scaling and GEMV in one launch
            return ops.awq_linear_row(x, self.inv_scale, self.w_codes, self.w_scales, self.w_zeros, self.bias,
                                      self.N, self.K)
        xh, xs = ops.awq_quant_act(x, self.inv_scale)
        return ops.awq_gemv(xh, xs, self.w_codes, self.w_scales, self.w_zeros, self.bias, M, self.N, self.K)

    __call__ = forward
