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
    or "mxfp4" (E2M1 codes, E8M0 scale per 32), as in the prepared dict."""

    def __init__(self, prepared: dict, bias: Optional[torch.Tensor], device):
        dev = torch.device(device)
        self.precision = prepared.get("precision", "int4")
        if self.precision not in ("int4", "mxfp4"):
            raise ValueError(f"unknown precision {self.precision!r}")
        self.K, self.N = prepared["K"], prepared["N"]
        self.rank, self.group = prepared["rank"], prepared["group"]
        self.smooth_inv = _to_dev(np.asarray(prepared["smooth_inv"], np.float32), dev)
        self.w_codes = _to_dev(np.asarray(prepared["w_codes"], np.uint8), dev)
        sdt = np.uint8 if self.precision == "mxfp4" else np.float16
        self.w_scales = _to_dev(np.asarray(prepared["w_scales"], sdt), dev)
        self.lora_down = _bits_to_bf16(prepared["lora_down"], dev) if self.rank else None
        self.lora_up = _bits_to_bf16(prepared["lora_up"], dev) if self.rank else None
        self.bias = None if bias is None else bias.detach().to(dev, torch.bfloat16).contiguous()

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, act_absmax, rank: int = 32, group: int = 64,
                    alpha: float = 0.5, device="cuda", precision: str = "int4"):
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
        return cls(prep, linear.bias, device)

    def forward(self, x: torch.Tensor, act: int = L.SVDQ_ACT_NONE, out_dtype: int = L.SVDQ_OUT_BF16):
        M = x.shape[0]
        if self.precision == "mxfp4":
            xc, xs, la = ops.quant_act_lora_down_mxfp4(x, self.smooth_inv, self.lora_down, self.rank, act)
            return ops.gemm_mxfp4_lora_up(xc, xs, self.w_codes, self.w_scales, la, self.lora_up, self.bias,
                                          M, self.N, self.K, self.rank, out_dtype)
        xc, xs, la = ops.quant_act_lora_down(x, self.smooth_inv, self.lora_down, self.rank, self.group, act)
        return ops.gemm_w4a4_lora_up(xc, xs, self.w_codes, self.w_scales, la, self.lora_up, self.bias,
                                     M, self.N, self.K, self.rank, self.group, out_dtype)

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
        xh, xs = ops.awq_quant_act(x, self.inv_scale)
        return ops.awq_gemv(xh, xs, self.w_codes, self.w_scales, self.w_zeros, self.bias, M, self.N, self.K)

    __call__ = forward
