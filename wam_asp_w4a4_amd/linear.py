"""A quantised linear module and an all-or-nothing installer.

The model card ("FastWAM UR3 3-task -- 4-bit quantisations", section
"Running the NVFP4 checkpoint") installs its NVFP4 deflated-ASP linears into a
model with one call that refuses to swap only part of the targets.  Here:

* ``ASPLinear`` holds one packed layer (``PackedLayer``) and applies it to an
  input of any leading shape (..., K); y has x's dtype (bfloat16 or float32).
* ``install(model, layers)`` replaces named ``torch.nn.Linear`` submodules by
  ``ASPLinear`` modules.  Every target is validated first -- the name resolves
  to an ``nn.Linear``, the packed layer's K and N equal its in/out features,
  its bias is present exactly when the Linear has one, it sits on the model's
  device -- and only when all of them pass is any module swapped.  Otherwise
  ``InstallError`` lists every problem and the model is left unchanged.

All arithmetic runs in libasp; this module only reshapes and dispatches.
"""

from __future__ import annotations

from typing import Mapping

import torch

from .layer import PackedLayer


class InstallError(ValueError):
    """Raised by install() before any module is swapped; .problems lists why."""

    def __init__(self, problems):
        super().__init__("install: no layer swapped:\n  " + "\n  ".join(problems))
        self.problems = list(problems)


class ASPLinear(torch.nn.Module):
    """y = the deflated-ASP NVFP4 layer applied to x (..., in_features).

    The packed weight, scales, low-rank factor, prep constants and bias are
    held as buffers of the packed layer (device tensors); the module has no
    trainable parameters.  Inputs in bfloat16 give bfloat16 outputs, float32
    inputs float32 outputs."""

    def __init__(self, packed: PackedLayer):
        super().__init__()
        self.packed = packed
        self.in_features = packed.K
        self.out_features = packed.N
        self.rank = packed.r

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, s, v, device=None, form: str = "deflated"):
        """Pack an nn.Linear's weight (and bias) with smoothing vector s (K) and
        basis v (K x r, or None for rank 0)."""
        w = linear.weight.detach().float().cpu().numpy()
        b = None if linear.bias is None else linear.bias.detach().float().cpu().numpy()
        dev = linear.weight.device if device is None else device
        return cls(PackedLayer.pack(w, s, v, b, dev, form=form))

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"x has {x.shape[-1]} features, the layer {self.in_features}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features).contiguous()
        y_dtype = "bf16" if x.dtype == torch.bfloat16 else "f32"
        y = self.packed.forward(x2, y_dtype)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"rank={self.rank}, bias={self.packed.bias is not None}, NVFP4 W4A4")


def _resolve(model: torch.nn.Module, name: str):
    """(parent module, attribute name, module) of a dotted submodule name."""
    parts = name.split(".")
    parent = model
    for p in parts[:-1]:
        parent = getattr(parent, p, None)
        if parent is None:
            return None, parts[-1], None
    return parent, parts[-1], getattr(parent, parts[-1], None)


def install(model: torch.nn.Module, layers: Mapping[str, PackedLayer]) -> list:
    """Swap every named nn.Linear of ``model`` for an ASPLinear of its packed
    layer, or none of them.  Returns the names swapped."""
    problems = []
    plan = []
    for name, packed in layers.items():
        parent, attr, mod = _resolve(model, name)
        if mod is None:
            problems.append(f"{name}: no such submodule")
            continue
        if not isinstance(mod, torch.nn.Linear):
            problems.append(f"{name}: a {type(mod).__name__}, not an nn.Linear")
            continue
        if not isinstance(packed, PackedLayer):
            problems.append(f"{name}: the packed layer is a {type(packed).__name__}")
            continue
        if (packed.K, packed.N) != (mod.in_features, mod.out_features):
            problems.append(f"{name}: packed {packed.K} -> {packed.N}, Linear "
                            f"{mod.in_features} -> {mod.out_features}")
        if (packed.bias is None) != (mod.bias is None):
            problems.append(f"{name}: bias {'missing' if packed.bias is None else 'unexpected'} "
                            "in the packed layer")
        if packed.device != mod.weight.device:
            problems.append(f"{name}: packed on {packed.device}, the Linear on {mod.weight.device}")
        plan.append((parent, attr, packed))
    if problems:
        raise InstallError(problems)
    for parent, attr, packed in plan:
        setattr(parent, attr, ASPLinear(packed))
    return list(layers)
