"""Prepared-layer checkpoints (safetensors + quantization_config header)."""
import json

import numpy as np
import pytest
import torch
from safetensors import safe_open
from safetensors.torch import save_file

import workloads

S = pytest.importorskip("w4a4_rank_corrected_svdq_amd")
from w4a4_rank_corrected_svdq_amd import checkpoint as C  # noqa: E402


def _layers(rank=32):
    wl = workloads.custom_workload(16, 256, 136, seed=61, n_out=3, bias=True)
    Lr = wl.layers[0]
    p = S.prepare_weights(Lr.weight_bits, wl.act_absmax(), rank=rank)
    return {"blocks.0.attn.to_q": p, "blocks.0.ff.proj": p}, {"blocks.0.attn.to_q": Lr.bias_bits}


@pytest.mark.parametrize("rank", [0, 32])
def test_round_trip_bit_exact(tmp_path, rank):
    layers, biases = _layers(rank)
    path = str(tmp_path / "m.safetensors")
    cfg = C.save_prepared(path, layers, biases)
    assert cfg["svdq_w4a4"] == {"precision": "int4", "group_size": 64, "rank": rank,
                                "targets": sorted(layers)}
    cfg2, got = C.load_prepared(path)
    assert cfg2 == cfg
    for name, p in layers.items():
        q, bias = got[name]
        for k in ("smooth_inv", "w_codes", "w_scales", "lora_down", "lora_up"):
            np.testing.assert_array_equal(np.asarray(q[k]), np.asarray(p[k]).reshape(q[k].shape))
        assert (q["K"], q["N"], q["rank"], q["group"]) == (p["K"], p["N"], p["rank"], p["group"])
        if name in biases:
            np.testing.assert_array_equal(bias, biases[name])
        else:
            assert bias is None


def test_header_is_plain_json_metadata(tmp_path):
    layers, biases = _layers()
    path = str(tmp_path / "m.safetensors")
    C.save_prepared(path, layers, biases)
    with safe_open(path, framework="pt") as f:
        meta = json.loads(f.metadata()["quantization_config"])
        assert f.get_tensor("blocks.0.ff.proj.lora_up").dtype == torch.bfloat16
    assert meta["quant_method"] == C.QUANT_METHOD and meta["compute_dtype"] == "bfloat16"


def _rewrite(path, out, mutate_cfg=None, drop=None, replace=None):
    with safe_open(path, framework="pt") as f:
        cfg = json.loads(f.metadata()["quantization_config"])
        t = {k: f.get_tensor(k) for k in f.keys()}
    if mutate_cfg:
        mutate_cfg(cfg)
    if drop:
        del t[drop]
    if replace:
        t[replace[0]] = replace[1]
    save_file(t, out, metadata={"quantization_config": json.dumps(cfg)})


@pytest.mark.parametrize("case", ["precision", "group", "rank", "missing", "shape", "dtype", "method"])
def test_load_rejects_inconsistent_files(tmp_path, case):
    layers, biases = _layers()
    path = str(tmp_path / "m.safetensors")
    bad = str(tmp_path / "bad.safetensors")
    C.save_prepared(path, layers, biases)
    if case == "precision":
        _rewrite(path, bad, lambda c: c["svdq_w4a4"].update(precision="nvfp4"))
    elif case == "group":
        _rewrite(path, bad, lambda c: c["svdq_w4a4"].update(group_size=16))
    elif case == "rank":
        _rewrite(path, bad, lambda c: c["svdq_w4a4"].update(rank=48))
    elif case == "missing":
        _rewrite(path, bad, drop="blocks.0.ff.proj.w_scales")
    elif case == "shape":
        _rewrite(path, bad, replace=("blocks.0.ff.proj.w_codes", torch.zeros((136, 64), dtype=torch.uint8)))
    elif case == "dtype":
        _rewrite(path, bad, replace=("blocks.0.ff.proj.w_scales", torch.zeros((4, 136), dtype=torch.float32)))
    elif case == "method":
        _rewrite(path, bad, lambda c: c.update(quant_method="other"))
    with pytest.raises(ValueError):
        C.load_prepared(bad)


def test_save_rejects_mixed_ranks(tmp_path):
    a, _ = _layers(32)
    b, _ = _layers(16)
    with pytest.raises(ValueError):
        C.save_prepared(str(tmp_path / "x.safetensors"), {"a": a["blocks.0.ff.proj"], "b": b["blocks.0.ff.proj"]})
