"""Prepared-layer checkpoints: a safetensors file whose metadata carries a
``quantization_config`` block.

The layout of the block follows the one the pages describe for quantized
Diffusers repositories ("Bringing Nunchaku 4-bit Diffusion Inference to
Diffusers", "Native loading in Diffusers"): a ``quant_method``, the
``compute_dtype`` and, per layer family, ``precision``, ``group_size``,
``rank`` and the list of ``targets`` (module names).  Here the family is
``svdq_w4a4`` with ``precision = "int4"``; each target stores the arrays the
kernels consume, in the ABI's storage layouts:

  <target>.smooth_inv  [K]        float32
  <target>.w_codes     [N][K/2]   uint8    (two INT4 codes per byte, low nibble = even k)
  <target>.w_scales    [K/64][N]  float16
  <target>.lora_down   [rank][K]  bfloat16 (absent when rank == 0)
  <target>.lora_up     [N][rank]  bfloat16 (absent when rank == 0)
  <target>.bias        [N]        bfloat16 (optional)

Loading reads only tensors and the JSON metadata string (no code is
executed from the file) and checks every shape against the header.
"""
from __future__ import annotations

import json
from typing import Dict, Optional, Tuple

import numpy as np
import torch
from safetensors import safe_open
from safetensors.torch import save_file

QUANT_METHOD = "svdq_w4a4_rank_corrected"
FAMILY = "svdq_w4a4"


def _bf16_from_bits(bits) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16).copy()).view(torch.bfloat16)


def _bits_from_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def save_prepared(path: str, layers: Dict[str, dict], biases: Optional[Dict[str, np.ndarray]] = None,
                  compute_dtype: str = "bfloat16") -> dict:
    """Write prepared layers (dicts as returned by ``prepare_weights``) and
    optional bias bit patterns (uint16 [N]) to ``path``.  All layers must
    share rank and group.  Returns the ``quantization_config`` written."""
    if not layers:
        raise ValueError("no layers to save")
    biases = biases or {}
    ranks = {int(p["rank"]) for p in layers.values()}
    groups = {int(p["group"]) for p in layers.values()}
    if len(ranks) != 1 or len(groups) != 1:
        raise ValueError("all layers of one checkpoint must share rank and group")
    rank, group = ranks.pop(), groups.pop()
    tensors = {}
    for name, p in layers.items():
        if "." in name and name.rsplit(".", 1)[1] in ("smooth_inv", "w_codes", "w_scales", "lora_down",
                                                      "lora_up", "bias"):
            raise ValueError(f"target name {name!r} ends in a reserved tensor suffix")
        # copies: one array may back several targets, and every tensor of a
        # safetensors file owns its storage
        tensors[f"{name}.smooth_inv"] = torch.from_numpy(np.array(p["smooth_inv"], np.float32))
        tensors[f"{name}.w_codes"] = torch.from_numpy(np.array(p["w_codes"], np.uint8))
        tensors[f"{name}.w_scales"] = torch.from_numpy(np.array(p["w_scales"], np.float16))
        if rank:
            tensors[f"{name}.lora_down"] = _bf16_from_bits(p["lora_down"])
            tensors[f"{name}.lora_up"] = _bf16_from_bits(p["lora_up"])
        if biases.get(name) is not None:
            tensors[f"{name}.bias"] = _bf16_from_bits(biases[name])
    config = {
        "quant_method": QUANT_METHOD,
        "compute_dtype": compute_dtype,
        FAMILY: {"precision": "int4", "group_size": group, "rank": rank, "targets": sorted(layers)},
    }
    save_file(tensors, path, metadata={"quantization_config": json.dumps(config)})
    return config


def read_config(path: str) -> dict:
    with safe_open(path, framework="pt") as f:
        meta = f.metadata() or {}
    if "quantization_config" not in meta:
        raise ValueError(f"{path}: no quantization_config in the file metadata")
    config = json.loads(meta["quantization_config"])
    fam = config.get(FAMILY)
    if config.get("quant_method") != QUANT_METHOD or not isinstance(fam, dict):
        raise ValueError(f"{path}: not an {QUANT_METHOD} checkpoint")
    if fam.get("precision") != "int4":
        raise ValueError(f"{path}: precision {fam.get('precision')!r} is not supported (int4 only)")
    if fam.get("group_size") != 64:
        raise ValueError(f"{path}: group_size {fam.get('group_size')!r} is not supported (64 only)")
    r = fam.get("rank")
    if not isinstance(r, int) or r < 0 or r % 16:
        raise ValueError(f"{path}: rank {r!r} is not a non-negative multiple of 16")
    if not isinstance(fam.get("targets"), list) or not fam["targets"]:
        raise ValueError(f"{path}: empty target list")
    return config


def load_prepared(path: str) -> Tuple[dict, Dict[str, Tuple[dict, Optional[np.ndarray]]]]:
    """Returns (quantization_config, {target: (prepared dict, bias bits or None)})
    with every shape checked against the header."""
    config = read_config(path)
    fam = config[FAMILY]
    rank, group = fam["rank"], fam["group_size"]
    out = {}
    with safe_open(path, framework="pt") as f:
        keys = set(f.keys())

        def get(name, dtype):
            if name not in keys:
                raise ValueError(f"{path}: missing tensor {name}")
            t = f.get_tensor(name)
            if t.dtype != dtype:
                raise ValueError(f"{path}: {name} has dtype {t.dtype}, expected {dtype}")
            return t

        for tgt in fam["targets"]:
            si = get(f"{tgt}.smooth_inv", torch.float32).numpy()
            wc = get(f"{tgt}.w_codes", torch.uint8).numpy()
            ws = get(f"{tgt}.w_scales", torch.float16).numpy()
            if si.ndim != 1 or wc.ndim != 2 or ws.ndim != 2:
                raise ValueError(f"{path}: {tgt}: wrong tensor ranks")
            K = si.shape[0]
            N = wc.shape[0]
            if K % group or wc.shape != (N, K // 2) or ws.shape != (K // group, N) or N % 8:
                raise ValueError(f"{path}: {tgt}: inconsistent shapes")
            if rank > min(K, N):
                raise ValueError(f"{path}: {tgt}: rank {rank} exceeds min(K, N)")
            p = dict(K=K, N=N, rank=rank, group=group, smooth_inv=si, w_codes=wc, w_scales=ws)
            if rank:
                ld = _bits_from_bf16(get(f"{tgt}.lora_down", torch.bfloat16))
                lu = _bits_from_bf16(get(f"{tgt}.lora_up", torch.bfloat16))
                if ld.shape != (rank, K) or lu.shape != (N, rank):
                    raise ValueError(f"{path}: {tgt}: low-rank factor shapes do not match rank {rank}")
                p["lora_down"], p["lora_up"] = ld, lu
            else:
                p["lora_down"] = np.zeros((0, K), np.uint16)
                p["lora_up"] = np.zeros((N, 0), np.uint16)
            bias = None
            if f"{tgt}.bias" in keys:
                bias = _bits_from_bf16(get(f"{tgt}.bias", torch.bfloat16))
                if bias.shape != (N,):
                    raise ValueError(f"{path}: {tgt}: bias shape {bias.shape} != ({N},)")
            out[tgt] = (p, bias)
    return config, out


def load_linears(path: str, device="cuda") -> Dict[str, "SVDQW4A4Linear"]:  # noqa: F821
    """Every target of the checkpoint as a device-resident ``SVDQW4A4Linear``."""
    from .linear import SVDQW4A4Linear
    _, layers = load_prepared(path)
    return {name: SVDQW4A4Linear(p, None if b is None else _bf16_from_bits(b), device)
            for name, (p, b) in layers.items()}
