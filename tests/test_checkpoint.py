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


def _mx_layers(rank=32):
    wl = workloads.custom_workload(16, 256, 136, seed=62, n_out=2, bias=True)
    p = S.prepare_weights_mxfp4(wl.layers[0].weight_bits, wl.act_absmax(), rank=rank)
    return {"blocks.1.attn.to_k": p}, {"blocks.1.attn.to_k": wl.layers[0].bias_bits}


def _awq_layers():
    wl = workloads.awq_workload(2, K=256, N=96, Mc=8, seed=63)
    p = S.awq_prepare(wl["weight_bits"], wl["x_cal_bits"])
    return {"blocks.0.norm1.linear": p}, wl["bias_bits"]


def _same(a, b):
    np.testing.assert_array_equal(np.asarray(a), np.asarray(b).reshape(np.asarray(a).shape))


@pytest.mark.parametrize("rank", [0, 32])
def test_round_trip_mxfp4(tmp_path, rank):
    layers, biases = _mx_layers(rank)
    path = str(tmp_path / "mx.safetensors")
    cfg = C.save_prepared(path, layers, biases)
    assert cfg["svdq_w4a4"] == {"precision": "mxfp4", "group_size": 32, "rank": rank,
                                "targets": ["blocks.1.attn.to_k"]}
    _, got = C.load_prepared(path)
    q, bias = got["blocks.1.attn.to_k"]
    p = layers["blocks.1.attn.to_k"]
    assert q["precision"] == "mxfp4" and q["w_scales"].dtype == np.uint8 and q["w_scales"].shape == (136, 8)
    for k in ("smooth_inv", "w_codes", "w_scales", "lora_down", "lora_up"):
        _same(q[k], p[k])
    _same(bias, biases["blocks.1.attn.to_k"])


def test_round_trip_awq_and_mixed_families(tmp_path):
    svdq, sb = _layers(32)
    awq, ab = _awq_layers()
    path = str(tmp_path / "mixed.safetensors")
    biases = dict(sb)
    biases["blocks.0.norm1.linear"] = ab
    cfg = C.save_prepared(path, svdq, biases, awq_layers=awq)
    assert cfg["awq_w4a16"] == {"precision": "int4", "group_size": 64, "targets": ["blocks.0.norm1.linear"]}
    assert cfg["svdq_w4a4"]["precision"] == "int4"
    _, got = C.load_prepared(path)
    assert set(got) == set(svdq) | set(awq)
    q, bias = got["blocks.0.norm1.linear"]
    p = awq["blocks.0.norm1.linear"]
    assert q["method"] == "awq_w4a16" and (q["K"], q["N"], q["group"]) == (256, 96, 64)
    for k in ("inv_scale", "w_codes", "w_scales", "w_zeros"):
        _same(q[k], p[k])
    _same(bias, biases["blocks.0.norm1.linear"])
    assert got["blocks.0.attn.to_q"][0]["method"] == "svdq_w4a4"
    # an AWQ-only file
    path2 = str(tmp_path / "awq.safetensors")
    cfg2 = C.save_prepared(path2, awq_layers=awq)
    assert "svdq_w4a4" not in cfg2
    _, got2 = C.load_prepared(path2)
    _same(got2["blocks.0.norm1.linear"][0]["w_zeros"], p["w_zeros"])


def test_save_rejects_unstorable_layers(tmp_path):
    a, _ = _layers(32)
    p = dict(a["blocks.0.ff.proj"])
    with pytest.raises(ValueError):            # int4 with a group other than 64
        C.save_prepared(str(tmp_path / "x.safetensors"), {"a": dict(p, group=128)})
    with pytest.raises(ValueError):            # unknown precision
        C.save_prepared(str(tmp_path / "x.safetensors"), {"a": dict(p, precision="nvfp4")})
    m, _ = _mx_layers(32)
    with pytest.raises(ValueError):            # mixed precisions in one family
        C.save_prepared(str(tmp_path / "x.safetensors"), {"a": p, "b": m["blocks.1.attn.to_k"]})
    awq, _ = _awq_layers()
    with pytest.raises(ValueError):            # one name in both families
        C.save_prepared(str(tmp_path / "x.safetensors"), {"n": p}, awq_layers={"n": awq["blocks.0.norm1.linear"]})
    with pytest.raises(ValueError):            # a bias for no target
        C.save_prepared(str(tmp_path / "x.safetensors"), {"a": p}, {"b": np.zeros(136, np.uint16)})
    with pytest.raises(ValueError):
        C.save_prepared(str(tmp_path / "x.safetensors"), {"a.w_zeros": p})


@pytest.mark.parametrize("case", ["mx_group", "mx_scales", "awq_group", "awq_zeros", "awq_missing"])
def test_load_rejects_bad_variant_files(tmp_path, case):
    path = str(tmp_path / "m.safetensors")
    bad = str(tmp_path / "bad.safetensors")
    if case.startswith("mx"):
        layers, biases = _mx_layers(32)
        C.save_prepared(path, layers, biases)
        if case == "mx_group":
            _rewrite(path, bad, lambda c: c["svdq_w4a4"].update(group_size=64))
        else:
            _rewrite(path, bad, replace=("blocks.1.attn.to_k.w_scales", torch.zeros((8, 136), dtype=torch.uint8)))
    else:
        awq, _ = _awq_layers()
        C.save_prepared(path, awq_layers=awq)
        if case == "awq_group":
            _rewrite(path, bad, lambda c: c["awq_w4a16"].update(group_size=128))
        elif case == "awq_zeros":
            _rewrite(path, bad, replace=("blocks.0.norm1.linear.w_zeros", torch.full((96, 4), 16, dtype=torch.uint8)))
        else:
            _rewrite(path, bad, drop="blocks.0.norm1.linear.inv_scale")
    with pytest.raises(ValueError):
        C.load_prepared(bad)
