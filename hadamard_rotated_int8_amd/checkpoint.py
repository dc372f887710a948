"""INT8 convrot safetensors checkpoints: load (and write) quantised linears.

Format, from the stable-diffusion.cpp page "INT8 Convrot Safetensors",
section "Checkpoint format": every quantised linear module ``<module>`` holds
  * ``<module>.weight``       int8 [out_features, in_features], used as stored
                              (no conversion at load time);
  * ``<module>.weight_scale`` one floating-point scale per output row, either
                              1-D [out] or ComfyUI's [out, 1], which is
                              normalised to 1-D here;
  * ``<module>.comfy_quant``  a uint8 tensor holding the module's quantisation
                              configuration as JSON, of the form
                              {"format": "int8_tensorwise", "convrot": true,
                               "convrot_groupsize": 256};
and, like any linear, optionally ``<module>.bias`` (converted to float32).
The group size must be a power of four dividing in_features.

Everything is validated on the host before anything is copied to a device;
a violation raises ``CheckpointError`` naming the module and the rule.  This
module does file IO and bookkeeping only; the weights go to the HIP library
as they are stored.  Files are read with the ``safetensors`` package, which
executes nothing from the file.
"""

from __future__ import annotations

import json
from dataclasses import dataclass

import numpy as np
import torch

SUPPORTED_FORMAT = "int8_tensorwise"
_FLOAT_DTYPES = (torch.float32, torch.float16, torch.bfloat16)


class CheckpointError(ValueError):
    """A tensor or configuration that the convrot format does not allow."""


@dataclass
class ConvrotModule:
    """One quantised linear as stored: codes, per-row scales, bias, config."""

    name: str
    q: torch.Tensor            # int8 [n, k]
    scale: torch.Tensor        # float32 [n]
    bias: torch.Tensor | None  # float32 [n] or None
    group_size: int
    config: dict

    @property
    def out_features(self) -> int:
        return int(self.q.shape[0])

    @property
    def in_features(self) -> int:
        return int(self.q.shape[1])


def _is_power_of_four(g: int) -> bool:
    return g >= 1 and (g & (g - 1)) == 0 and (g.bit_length() - 1) % 2 == 0


def parse_config(raw, module: str = "?") -> dict:
    """Decode and check a ``comfy_quant`` configuration (uint8 tensor, bytes or str)."""
    if isinstance(raw, torch.Tensor):
        if raw.dtype != torch.uint8 or raw.dim() != 1:
            raise CheckpointError(f"{module}.comfy_quant must be a 1-D uint8 tensor")
        raw = bytes(raw.cpu().numpy().tobytes())
    if isinstance(raw, (bytes, bytearray)):
        try:
            raw = raw.decode("utf-8")
        except UnicodeDecodeError as e:
            raise CheckpointError(f"{module}.comfy_quant is not UTF-8 text") from e
    try:
        cfg = json.loads(raw)
    except json.JSONDecodeError as e:
        raise CheckpointError(f"{module}.comfy_quant is not valid JSON: {e}") from e
    if not isinstance(cfg, dict):
        raise CheckpointError(f"{module}.comfy_quant must be a JSON object")
    if cfg.get("format") != SUPPORTED_FORMAT:
        raise CheckpointError(f"{module}: format {cfg.get('format')!r} is not {SUPPORTED_FORMAT!r}")
    if cfg.get("convrot") is not True:
        raise CheckpointError(f"{module}: convrot must be true (only rotated weights are supported)")
    g = cfg.get("convrot_groupsize")
    if isinstance(g, bool) or not isinstance(g, int) or not _is_power_of_four(g):
        raise CheckpointError(f"{module}: convrot_groupsize {g!r} is not a power of four")
    return cfg


def _module(name: str, tensors: dict) -> ConvrotModule:
    w = tensors.get(name + ".weight")
    s = tensors.get(name + ".weight_scale")
    cq = tensors.get(name + ".comfy_quant")
    if w is None or s is None or cq is None:
        missing = [t for t, v in (("weight", w), ("weight_scale", s), ("comfy_quant", cq)) if v is None]
        raise CheckpointError(f"{name}: missing {', '.join(missing)}")
    cfg = parse_config(cq, name)
    if w.dtype != torch.int8 or w.dim() != 2:
        raise CheckpointError(f"{name}.weight must be a 2-D int8 tensor, got {w.dtype} {tuple(w.shape)}")
    n, k = w.shape
    if w.numel() and int(w.min()) < -127:
        # The page's section "Weight quantization" clamps codes to [-127, 127];
        # -128 would also break the int32 range the GEMM's K limit is sized for.
        raise CheckpointError(f"{name}.weight holds the code -128, outside [-127, 127]")
    if s.dtype not in _FLOAT_DTYPES:
        raise CheckpointError(f"{name}.weight_scale must be floating point, got {s.dtype}")
    if tuple(s.shape) == (n, 1):
        s = s.reshape(n)  # ComfyUI's [out_features, 1]
    if tuple(s.shape) != (n,):
        raise CheckpointError(f"{name}.weight_scale has shape {tuple(s.shape)}, expected ({n},) or ({n}, 1)")
    g = int(cfg["convrot_groupsize"])
    if k % g != 0:
        raise CheckpointError(f"{name}: convrot_groupsize {g} does not divide in_features {k}")
    b = tensors.get(name + ".bias")
    if b is not None:
        if b.dtype not in _FLOAT_DTYPES or tuple(b.shape) != (n,):
            raise CheckpointError(f"{name}.bias must be a floating-point ({n},) tensor")
        b = b.to(torch.float32)
    s32 = s.to(torch.float32)
    if not bool(torch.isfinite(s32).all()) or bool((s32 < 0).any()):
        raise CheckpointError(f"{name}.weight_scale must be finite and non-negative")
    return ConvrotModule(name, w.contiguous(), s32.contiguous(), None if b is None else b.contiguous(),
                         g, cfg)


def read_modules(tensors: dict) -> dict:
    """All convrot modules of a name -> tensor mapping (CPU tensors), validated."""
    names = sorted(key[: -len(".comfy_quant")] for key in tensors if key.endswith(".comfy_quant"))
    return {name: _module(name, tensors) for name in names}


def load_checkpoint(path: str, device=None) -> dict:
    """Read every convrot module of a safetensors file.

    Returns {module name: ConvrotModule}; with ``device`` set, the tensors are
    copied there after all modules have been validated.  Tensors that belong
    to no convrot module are ignored.
    """
    from safetensors.torch import load_file

    mods = read_modules(load_file(path, device="cpu"))
    if device is not None:
        for m in mods.values():
            m.q = m.q.to(device)
            m.scale = m.scale.to(device)
            if m.bias is not None:
                m.bias = m.bias.to(device)
    return mods


def to_weights(module: ConvrotModule):
    """The module as the binding's QuantizedWeights (device tensors, stored codes)."""
    from . import QuantizedWeights

    if not module.q.is_cuda:
        raise ValueError(f"{module.name}: load the checkpoint with device='cuda' first")
    return QuantizedWeights(module.q, module.scale, module.bias, module.group_size)


def save_checkpoint(path: str, modules: dict, scale_2d: bool = True) -> None:
    """Write modules {name: (q int8 [n,k], scale [n], bias [n] or None, group_size)}.

    Scales are written as ComfyUI's [n, 1] float32 when ``scale_2d`` is set.
    The codes are written as given (quantise them with
    ``quantize_weights`` first).
    """
    from safetensors.torch import save_file

    out = {}
    for name, (q, s, b, g) in modules.items():
        q = torch.as_tensor(np.asarray(q) if not isinstance(q, torch.Tensor) else q).cpu()
        s = torch.as_tensor(np.asarray(s) if not isinstance(s, torch.Tensor) else s).cpu()
        if q.dtype != torch.int8 or q.dim() != 2:
            raise CheckpointError(f"{name}: codes must be int8 [n, k]")
        cfg = {"format": SUPPORTED_FORMAT, "convrot": True, "convrot_groupsize": int(g)}
        parse_config(json.dumps(cfg), name)
        if q.shape[1] % int(g) != 0:
            raise CheckpointError(f"{name}: group size {g} does not divide in_features {q.shape[1]}")
        s = s.to(torch.float32).reshape(-1)
        out[name + ".weight"] = q.contiguous()
        out[name + ".weight_scale"] = (s.reshape(-1, 1) if scale_2d else s).contiguous()
        out[name + ".comfy_quant"] = torch.frombuffer(bytearray(json.dumps(cfg).encode()),
                                                      dtype=torch.uint8).clone()
        if b is not None:
            bt = torch.as_tensor(np.asarray(b) if not isinstance(b, torch.Tensor) else b).cpu()
            out[name + ".bias"] = bt.to(torch.float32).reshape(-1).contiguous()
    save_file(out, path)
