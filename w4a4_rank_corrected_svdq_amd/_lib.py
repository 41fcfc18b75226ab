"""ctypes loader for ``libsvdq.so`` (the C ABI declared in include/svdq.h).

There is no fallback: if the library is missing or cannot be loaded, every
entry point raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvdq.so")

SVDQ_OK = 0
SVDQ_ERR_INVALID_ARG = -1
SVDQ_ERR_UNSUPPORTED_SHAPE = -2
SVDQ_ERR_UNSUPPORTED_DEVICE = -3
SVDQ_ERR_HIP = -4
SVDQ_ERR_NUMERIC = -5
SVDQ_ACT_NONE = 0
SVDQ_ACT_GELU_TANH = 1
SVDQ_OUT_BF16 = 0
SVDQ_OUT_F32 = 1
SVDQ_GROUP = 64
SVDQ_MAX_RANK = 256
SVDQ_FP6_ACTIVATIONS = 0
SVDQ_FP6_WEIGHTS = 1
SVDQ_CHAIN_SCRATCH_BYTES = 32 << 20
SVDQ_AWQ_MAX_ROWS = 16
SVDQ_AWQ_ROW_MAX_K = 8192

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float

# name -> (restype, argtypes); every function declared in include/*.h
SIGNATURES = {
    "svdq_status_string": (ctypes.c_char_p, [_i]),
    "svdq_version": (_i, []),
    "svdq_device_check": (_i, [_i]),
    "svdq_prepared_bytes": (_i, [_i, _i, _i, _i, ctypes.POINTER(ctypes.c_size_t)]),
    "svdq_prepare_weights": (_i, [_p, _i, _i, _p, _f, _i, _i, _p, _p, _p, _p, _p]),
    "svdq_prepare_weights_ex": (_i, [_p, _i, _i, _p, _f, _i, _i, _p, _p, _i, ctypes.c_uint64,
                                     _p, _p, _p, _p, _p, _p]),
    "svdq_quant_act_lora_down": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p]),
    "svdq_gemm_w4a4_lora_up": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p]),
    "svdq_lora_down": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _p, _p]),
    "svdq_lora_up_add": (_i, [_p, _p, _i, _i, _i, _p, _p]),
    "svdq_gemm_w4a4_lora_up_qkv": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_float,
                                        _i, _i, _i, _i, _i, _i, _p, _p]),
    "svdq_awq_prepare": (_i, [_p, _i, _i, _p, _i, ctypes.c_double, _i, _p, _p, _p, _p, _p]),
    "svdq_awq_quant_act": (_i, [_p, _p, _i, _i, _p, _p, _p]),
    "svdq_awq_gemv": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _p, _p]),
    "svdq_awq_linear_row": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _p, _p]),
    "svdq_prepared_bytes_mxfp4": (_i, [_i, _i, _i, ctypes.POINTER(ctypes.c_size_t)]),
    "svdq_prepare_weights_mxfp4": (_i, [_p, _i, _i, _p, ctypes.c_float, _i, _p, _p, _i, ctypes.c_uint64,
                                        _p, _p, _p, _p, _p, _p]),
    "svdq_quant_act_lora_down_mxfp4": (_i, [_p, _p, _p, _i, _i, _i, _i, _p, _p, _p, _p]),
    "svdq_gemm_mxfp4_lora_up": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p]),
    "svdq_fp6_operand_bytes": (_i, [_i, _i, _i, ctypes.POINTER(ctypes.c_size_t)]),
    "svdq_pack_fp6_operand": (_i, [_p, _i, _i, _i, _p]),
    "svdq_quant_act_lora_down_fp6": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p]),
    "svdq_gemm_w4a4_fp6_lora_up": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p]),
    "svdq_gemm_w4a4_fp6_lora_up_n192": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p]),
    "svdq_fp6_n192_preferred": (_i, [_i, _i]),
    "svdq_int4_route": (_i, [_i, _i]),
    "svdq_gemm_w4a4_fp6_lora_up_qkv": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_float,
                                            _i, _i, _i, _i, _i, _i, _p, _p]),
    "svdq_mlp_chain_workspace_bytes": (_i, [_i, _i, _i, ctypes.POINTER(ctypes.c_size_t)]),
    "svdq_gemm_w4a4_fp6_mlp_chain": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i,
                                          _p, _p, _i, _p, _p, _p, _p, ctypes.c_size_t, _p]),
    "svdq_gemm_w4a4_fp6_mlp_chain_noalloc": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i,
                                                  _p, _p, _i, _p, _p, _p, _p]),
    # include/svdq_probe.h (benchmark harness)
    "svdq_probe_mfma": (_i, [_i, _i, _i, _p, _p]),
    "svdq_probe_mfma_ops": (ctypes.c_double, [_i, _i, _i]),
}
SVDQ_PROBE_MFMA_I8 = 0
SVDQ_PROBE_MFMA_FP4 = 1
SVDQ_PROBE_MFMA_FP6 = 2
SVDQ_PROBE_DEQUANT = 3
SVDQ_PROBE_FP6_DEQUANT = 4


class SVDQError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = status_string(status)
        super().__init__(f"{what}: {msg}" if what else msg)


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m w4a4_rank_corrected_svdq_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().svdq_status_string(int(status)).decode()


def check(status: int, what: str = "") -> None:
    if status != SVDQ_OK:
        raise SVDQError(status, what)
