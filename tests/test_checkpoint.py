"""The INT8 convrot safetensors loader (host side; no GPU needed).

The format is the one the stable-diffusion.cpp page "INT8 Convrot
Safetensors" describes in its section "Checkpoint format"; the synthetic
files here are quantised by the oracle, so every stored value is known.
"""

import json
import os

import numpy as np
import pytest
import torch
from safetensors.torch import save_file

from hadamard_rotated_int8_amd import checkpoint as ck
from oracle import convrot_oracle as orc


def _quantised(n, k, g, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    q, s = orc.quantize_weights(w, g)
    b = (rng.standard_normal(n) * 0.01).astype(np.float32)
    return q, s, b


def test_page_config_parses(golden_dir):
    """The configuration printed on the page is accepted, group size 256."""
    raw = open(os.path.join(golden_dir, "comfy_quant_h256.json")).read()
    cfg = ck.parse_config(raw)
    assert cfg["convrot_groupsize"] == 256 and cfg["convrot"] is True


@pytest.mark.parametrize("scale_2d", [True, False])
def test_round_trip(tmp_path, scale_2d):
    mods = {"blocks.0.attn.qkv": _quantised(96, 512, 256, 1) + (256,),
            "blocks.0.mlp.fc1": _quantised(64, 256, 16, 2) + (16,)}
    mods["blocks.0.mlp.fc1"] = mods["blocks.0.mlp.fc1"][:2] + (None, 16)  # no bias
    path = str(tmp_path / "m.safetensors")
    ck.save_checkpoint(path, mods, scale_2d=scale_2d)
    got = ck.load_checkpoint(path)
    assert sorted(got) == sorted(mods)
    for name, (q, s, b, g) in mods.items():
        m = got[name]
        assert m.q.dtype == torch.int8 and np.array_equal(m.q.numpy(), q)
        assert m.scale.dtype == torch.float32 and m.scale.shape == (q.shape[0],)
        assert np.array_equal(m.scale.numpy(), s)
        assert m.group_size == g and m.in_features == q.shape[1]
        if b is None:
            assert m.bias is None
        else:
            assert np.array_equal(m.bias.numpy(), b)


def test_comfyui_layouts_and_dtypes(tmp_path):
    """[out, 1] scales become 1-D; bf16 / fp16 scales and biases become float32;
    tensors of no convrot module are ignored."""
    q, s, b = _quantised(8, 64, 64, 3)
    cfg = torch.frombuffer(bytearray(json.dumps(
        {"format": "int8_tensorwise", "convrot": True, "convrot_groupsize": 64}).encode()),
        dtype=torch.uint8).clone()
    path = str(tmp_path / "c.safetensors")
    save_file({"l.weight": torch.from_numpy(q), "l.weight_scale": torch.from_numpy(s).to(torch.bfloat16).reshape(8, 1),
               "l.comfy_quant": cfg, "l.bias": torch.from_numpy(b).to(torch.float16),
               "norm.weight": torch.ones(64)}, path)
    m = ck.load_checkpoint(path)["l"]
    assert m.scale.shape == (8,) and m.scale.dtype == torch.float32
    assert np.array_equal(m.scale.numpy(), torch.from_numpy(s).to(torch.bfloat16).float().numpy())
    assert m.bias.dtype == torch.float32
    assert list(ck.load_checkpoint(path)) == ["l"]


def _write(tmp_path, tensors):
    path = str(tmp_path / "bad.safetensors")
    save_file(tensors, path)
    return path


def _cfg(**kw):
    c = {"format": "int8_tensorwise", "convrot": True, "convrot_groupsize": 16}
    c.update(kw)
    return torch.frombuffer(bytearray(json.dumps(c).encode()), dtype=torch.uint8).clone()


@pytest.mark.parametrize("case", ["missing_scale", "float_weight", "bad_json", "format", "no_convrot",
                                  "group_not_pow4", "group_bool", "group_not_dividing",
                                  "scale_shape", "negative_scale", "bias_shape", "code_minus_128"])
def test_rejections(tmp_path, case):
    q = torch.zeros((4, 32), dtype=torch.int8)
    t = {"m.weight": q, "m.weight_scale": torch.ones(4), "m.comfy_quant": _cfg()}
    if case == "missing_scale":
        del t["m.weight_scale"]
    elif case == "float_weight":
        t["m.weight"] = torch.zeros((4, 32))
    elif case == "bad_json":
        t["m.comfy_quant"] = torch.frombuffer(bytearray(b"{not json"), dtype=torch.uint8).clone()
    elif case == "format":
        t["m.comfy_quant"] = _cfg(format="float8_e4m3fn")
    elif case == "no_convrot":
        t["m.comfy_quant"] = _cfg(convrot=False)
    elif case == "group_not_pow4":
        t["m.comfy_quant"] = _cfg(convrot_groupsize=8)
    elif case == "group_bool":
        t["m.comfy_quant"] = _cfg(convrot_groupsize=True)
    elif case == "group_not_dividing":
        t["m.comfy_quant"] = _cfg(convrot_groupsize=64)
    elif case == "scale_shape":
        t["m.weight_scale"] = torch.ones(5)
    elif case == "negative_scale":
        t["m.weight_scale"] = -torch.ones(4)
    elif case == "bias_shape":
        t["m.bias"] = torch.ones(3)
    elif case == "code_minus_128":
        q = q.clone()
        q[2, 7] = -128
        t["m.weight"] = q
    with pytest.raises(ck.CheckpointError):
        ck.load_checkpoint(_write(tmp_path, t))


def test_group_size_rule():
    """Powers of four only (1, 4, 16, ...), as the format section requires."""
    assert [g for g in range(1, 300) if ck._is_power_of_four(g)] == [1, 4, 16, 64, 256]
