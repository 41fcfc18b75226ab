"""Prepared-layer checkpoints: a safetensors file whose metadata carries a
``quantization_config`` block.

The layout of the block follows the one the pages describe for quantized
Diffusers repositories ("Bringing Nunchaku 4-bit Diffusion Inference to
Diffusers", "Native loading in Diffusers"; "Introducing Nunchaku Lite" for the
second family): a ``quant_method``, the ``compute_dtype`` and, per layer
family, its ``precision``, ``group_size``, ``rank`` and the list of
``targets`` (module names).  Two families, each optional but not both absent:

``svdq_w4a4`` (attention and feed-forward projections), precision "int4"
(group 64) or "mxfp4" (group 32); per target, in the ABI's storage layouts:

  <target>.smooth_inv  [K]        float32
  <target>.w_codes     [N][K/2]   uint8    (two 4-bit codes per byte, low nibble = even k)
  <target>.w_scales    [K/64][N]  float16  (int4)   or  [N][K/32] uint8 E8M0 (mxfp4)
  <target>.lora_down   [rank][K]  bfloat16 (absent when rank == 0)
  <target>.lora_up     [N][rank]  bfloat16 (absent when rank == 0)
  <target>.bias        [N]        bfloat16 (optional)

``awq_w4a16`` (the modulation projections), precision "int4", group 64, no
rank; per target:

  <target>.inv_scale   [K]        float32  (1 / activation-aware channel scale)
  <target>.w_codes     [N][K/2]   uint8    (unsigned codes 0..15, low nibble = even k)
  <target>.w_scales    [N][K/64]  float16
  <target>.w_zeros     [N][K/64]  uint8
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
AWQ_FAMILY = "awq_w4a16"
SVDQ_GROUP = {"int4": 64, "mxfp4": 32}
_SUFFIXES = ("smooth_inv", "inv_scale", "w_codes", "w_scales", "w_zeros", "lora_down", "lora_up", "bias")


def _bf16_from_bits(bits) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16).copy()).view(torch.bfloat16)


def _bits_from_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def _check_name(name: str) -> None:
    if "." in name and name.rsplit(".", 1)[1] in _SUFFIXES:
        raise ValueError(f"target name {name!r} ends in a reserved tensor suffix")


def save_prepared(path: str, layers: Optional[Dict[str, dict]] = None,
                  biases: Optional[Dict[str, np.ndarray]] = None, compute_dtype: str = "bfloat16",
                  awq_layers: Optional[Dict[str, dict]] = None) -> dict:
    """Write prepared layers and optional bias bit patterns (uint16 [N], keyed
    by target) to ``path``.  ``layers`` are dicts as returned by
    ``prepare_weights`` or ``prepare_weights_mxfp4`` (all of one precision,
    rank and group); ``awq_layers`` dicts as returned by ``awq_prepare``.
    Returns the ``quantization_config`` written."""
    layers, awq_layers, biases = layers or {}, awq_layers or {}, biases or {}
    if not layers and not awq_layers:
        raise ValueError("no layers to save")
    if set(layers) & set(awq_layers):
        raise ValueError("a target name appears in both families")
    tensors = {}
    config = {"quant_method": QUANT_METHOD, "compute_dtype": compute_dtype}
    if layers:
        precs = {p.get("precision", "int4") for p in layers.values()}
        ranks = {int(p["rank"]) for p in layers.values()}
        groups = {int(p["group"]) for p in layers.values()}
        if len(ranks) != 1 or len(groups) != 1 or len(precs) != 1:
            raise ValueError("all svdq_w4a4 layers of one checkpoint must share precision, rank and group")
        prec, rank, group = precs.pop(), ranks.pop(), groups.pop()
        if SVDQ_GROUP.get(prec) != group:
            raise ValueError(f"precision {prec!r} with group {group} cannot be stored "
                             f"(int4 uses group 64, mxfp4 group 32)")
        sdt = np.float16 if prec == "int4" else np.uint8
        for name, p in layers.items():
            _check_name(name)
            K, N = int(p["K"]), int(p["N"])
            sshape = (K // 64, N) if prec == "int4" else (N, K // 32)
            # copies: one array may back several targets, and every tensor of
            # a safetensors file owns its storage
            tensors[f"{name}.smooth_inv"] = torch.from_numpy(np.array(p["smooth_inv"], np.float32).reshape(K))
            tensors[f"{name}.w_codes"] = torch.from_numpy(np.array(p["w_codes"], np.uint8).reshape(N, K // 2))
            tensors[f"{name}.w_scales"] = torch.from_numpy(np.array(p["w_scales"], sdt).reshape(sshape))
            if rank:
                tensors[f"{name}.lora_down"] = _bf16_from_bits(np.asarray(p["lora_down"]).reshape(rank, K))
                tensors[f"{name}.lora_up"] = _bf16_from_bits(np.asarray(p["lora_up"]).reshape(N, rank))
        config[FAMILY] = {"precision": prec, "group_size": group, "rank": rank, "targets": sorted(layers)}
    if awq_layers:
        if {int(p["group"]) for p in awq_layers.values()} != {64}:
            raise ValueError("awq_w4a16 layers are stored with group 64 only")
        for name, p in awq_layers.items():
            _check_name(name)
            K, N = int(p["K"]), int(p["N"])
            tensors[f"{name}.inv_scale"] = torch.from_numpy(np.array(p["inv_scale"], np.float32).reshape(K))
            tensors[f"{name}.w_codes"] = torch.from_numpy(np.array(p["w_codes"], np.uint8).reshape(N, K // 2))
            tensors[f"{name}.w_scales"] = torch.from_numpy(np.array(p["w_scales"], np.float16).reshape(N, K // 64))
            tensors[f"{name}.w_zeros"] = torch.from_numpy(np.array(p["w_zeros"], np.uint8).reshape(N, K // 64))
        config[AWQ_FAMILY] = {"precision": "int4", "group_size": 64, "targets": sorted(awq_layers)}
    for name, b in biases.items():
        if name not in layers and name not in awq_layers:
            raise ValueError(f"bias for unknown target {name!r}")
        if b is not None:
            tensors[f"{name}.bias"] = _bf16_from_bits(b)
    save_file(tensors, path, metadata={"quantization_config": json.dumps(config)})
    return config


def _check_targets(path, fam, name):
    t = fam.get("targets")
    if not isinstance(t, list) or not t or not all(isinstance(x, str) for x in t):
        raise ValueError(f"{path}: {name}: empty or malformed target list")


def read_config(path: str) -> dict:
    with safe_open(path, framework="pt") as f:
        meta = f.metadata() or {}
    if "quantization_config" not in meta:
        raise ValueError(f"{path}: no quantization_config in the file metadata")
    config = json.loads(meta["quantization_config"])
    if config.get("quant_method") != QUANT_METHOD:
        raise ValueError(f"{path}: not an {QUANT_METHOD} checkpoint")
    fam, awq = config.get(FAMILY), config.get(AWQ_FAMILY)
    if fam is None and awq is None:
        raise ValueError(f"{path}: neither a {FAMILY} nor an {AWQ_FAMILY} block")
    if fam is not None:
        if not isinstance(fam, dict):
            raise ValueError(f"{path}: malformed {FAMILY} block")
        prec = fam.get("precision")
        if prec not in SVDQ_GROUP:
            raise ValueError(f"{path}: precision {prec!r} is not supported (int4 or mxfp4)")
        if fam.get("group_size") != SVDQ_GROUP[prec]:
            raise ValueError(f"{path}: group_size {fam.get('group_size')!r} does not match precision {prec}")
        r = fam.get("rank")
        if not isinstance(r, int) or r < 0 or r % 16:
            raise ValueError(f"{path}: rank {r!r} is not a non-negative multiple of 16")
        _check_targets(path, fam, FAMILY)
    if awq is not None:
        if not isinstance(awq, dict) or awq.get("precision") != "int4" or awq.get("group_size") != 64:
            raise ValueError(f"{path}: {AWQ_FAMILY} supports precision int4 with group 64 only")
        _check_targets(path, awq, AWQ_FAMILY)
    if fam is not None and awq is not None and set(fam["targets"]) & set(awq["targets"]):
        raise ValueError(f"{path}: a target appears in both families")
    return config


def load_prepared(path: str) -> Tuple[dict, Dict[str, Tuple[dict, Optional[np.ndarray]]]]:
    """Returns (quantization_config, {target: (prepared dict, bias bits or
    None)}) with every shape checked against the header.  The prepared dicts
    carry ``method`` ("svdq_w4a4" or "awq_w4a16") and, for the first family,
    ``precision``."""
    config = read_config(path)
    out = {}
    with safe_open(path, framework="pt") as f:
        keys = set(f.keys())

        def get(name, dtype, shape):
            if name not in keys:
                raise ValueError(f"{path}: missing tensor {name}")
            t = f.get_tensor(name)
            if t.dtype != dtype:
                raise ValueError(f"{path}: {name} has dtype {t.dtype}, expected {dtype}")
            if shape is not None and tuple(t.shape) != tuple(shape):
                raise ValueError(f"{path}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
            return t

        def bias_of(tgt, N):
            if f"{tgt}.bias" not in keys:
                return None
            return _bits_from_bf16(get(f"{tgt}.bias", torch.bfloat16, (N,)))

        fam = config.get(FAMILY)
        if fam is not None:
            prec, rank, group = fam["precision"], fam["rank"], fam["group_size"]
            for tgt in fam["targets"]:
                si = get(f"{tgt}.smooth_inv", torch.float32, None).numpy()
                wc = get(f"{tgt}.w_codes", torch.uint8, None).numpy()
                if si.ndim != 1 or wc.ndim != 2:
                    raise ValueError(f"{path}: {tgt}: wrong tensor ranks")
                K, N = si.shape[0], wc.shape[0]
                if K % 64 or wc.shape != (N, K // 2) or N % 8:
                    raise ValueError(f"{path}: {tgt}: inconsistent shapes")
                if prec == "int4":
                    ws = get(f"{tgt}.w_scales", torch.float16, (K // 64, N)).numpy()
                else:
                    ws = get(f"{tgt}.w_scales", torch.uint8, (N, K // 32)).numpy()
                if rank > min(K, N):
                    raise ValueError(f"{path}: {tgt}: rank {rank} exceeds min(K, N)")
                p = dict(K=K, N=N, rank=rank, group=group, precision=prec, method=FAMILY,
                         smooth_inv=si, w_codes=wc, w_scales=ws)
                if rank:
                    p["lora_down"] = _bits_from_bf16(get(f"{tgt}.lora_down", torch.bfloat16, (rank, K)))
                    p["lora_up"] = _bits_from_bf16(get(f"{tgt}.lora_up", torch.bfloat16, (N, rank)))
                else:
                    p["lora_down"] = np.zeros((0, K), np.uint16)
                    p["lora_up"] = np.zeros((N, 0), np.uint16)
                out[tgt] = (p, bias_of(tgt, N))
        awq = config.get(AWQ_FAMILY)
        if awq is not None:
            for tgt in awq["targets"]:
                inv = get(f"{tgt}.inv_scale", torch.float32, None).numpy()
                wc = get(f"{tgt}.w_codes", torch.uint8, None).numpy()
                if inv.ndim != 1 or wc.ndim != 2:
                    raise ValueError(f"{path}: {tgt}: wrong tensor ranks")
                K, N = inv.shape[0], wc.shape[0]
                if K % 64 or wc.shape != (N, K // 2):
                    raise ValueError(f"{path}: {tgt}: inconsistent shapes")
                p = dict(K=K, N=N, group=64, method=AWQ_FAMILY, inv_scale=inv, w_codes=wc,
                         w_scales=get(f"{tgt}.w_scales", torch.float16, (N, K // 64)).numpy(),
                         w_zeros=get(f"{tgt}.w_zeros", torch.uint8, (N, K // 64)).numpy())
                if p["w_zeros"].max(initial=0) > 15:
                    raise ValueError(f"{path}: {tgt}: zero point above 15")
                out[tgt] = (p, bias_of(tgt, N))
    return config, out


def load_linears(path: str, device="cuda") -> dict:
    """Every target of the checkpoint as a device-resident layer:
    ``SVDQW4A4Linear`` for the svdq_w4a4 family, ``AWQW4A16Linear`` for
    awq_w4a16."""
    from .linear import AWQW4A16Linear, SVDQW4A4Linear
    _, layers = load_prepared(path)
    out = {}
    for name, (p, b) in layers.items():
        bias = None if b is None else _bf16_from_bits(b)
        cls = AWQW4A16Linear if p["method"] == AWQ_FAMILY else SVDQW4A4Linear
        out[name] = cls(p, bias, device)
    return out
