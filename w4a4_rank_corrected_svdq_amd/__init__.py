"""SVDQuant W4A4 linear with a rank-r 16-bit branch, native to MI355X (gfx950).

The compute lives in ``libsvdq.so`` (C ABI in ``include/svdq.h``); this
package is its Python binding.
"""
from ._lib import SVDQError, lib  # noqa: F401
from . import _lib as abi  # noqa: F401
from .ops import (awq_gemv, awq_linear_row, awq_prepare, awq_quant_act, device_check, gemm_mxfp4_lora_up, gemm_w4a4_lora_up, gemm_w4a4_lora_up_qkv,  # noqa: F401
                  fp6_operand_bytes, gemm_w4a4_fp6_lora_up, gemm_w4a4_fp6_lora_up_n192, gemm_w4a4_fp6_lora_up_qkv, fp6_n192_preferred, int4_route, gemm_w4a4_fp6_mlp_chain, lora_down,
                  mlp_chain_workspace_bytes, pack_fp6_operand,
                  quant_act_lora_down_fp6,
                  lora_up_add, prepare_weights, prepare_weights_mxfp4, prepared_bytes,
                  prepared_bytes_mxfp4, quant_act_lora_down, quant_act_lora_down_mxfp4)
from .linear import AWQW4A16Linear, SVDQMLPChain, SVDQW4A4Linear  # noqa: F401
from .checkpoint import load_linears, load_prepared, save_prepared  # noqa: F401

__version__ = "0.1.0"
