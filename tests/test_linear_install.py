"""ASPLinear and the all-or-nothing install (CPU: validation and swapping only;
no call here reaches a kernel), and the input checks of the packed layer that
run before any launch.

The model card ("FastWAM UR3 3-task -- 4-bit quantisations", section "Running
the NVFP4 checkpoint") states that its installer raises rather than swapping a
subset of the targets; install() here follows that."""

import numpy as np
import pytest
import torch

from wam_asp_w4a4_amd import synth
from wam_asp_w4a4_amd.layer import PackedLayer
from wam_asp_w4a4_amd.linear import ASPLinear, InstallError, install


def _packed(K, N, r, bias=True, seed=0):
    lay = synth.make_layer("p", 8, K, N, r, seed=seed, dtype="f32")
    return PackedLayer.pack(lay.w, lay.s, lay.v, lay.b if bias else None, "cpu")


class Block(torch.nn.Module):
    def __init__(self):
        super().__init__()
        self.q = torch.nn.Linear(256, 128)
        self.o = torch.nn.Linear(128, 256, bias=False)
        self.ffn = torch.nn.Sequential(torch.nn.Linear(256, 384), torch.nn.GELU(),
                                       torch.nn.Linear(384, 256))


def test_install_swaps_every_target():
    m = Block()
    done = install(m, {"q": _packed(256, 128, 32), "o": _packed(128, 256, 0, bias=False),
                       "ffn.0": _packed(256, 384, 16), "ffn.2": _packed(384, 256, 32)})
    assert done == ["q", "o", "ffn.0", "ffn.2"]
    assert isinstance(m.q, ASPLinear) and isinstance(m.o, ASPLinear)
    assert isinstance(m.ffn[0], ASPLinear) and isinstance(m.ffn[2], ASPLinear)
    assert isinstance(m.ffn[1], torch.nn.GELU)
    assert (m.q.in_features, m.q.out_features, m.q.rank) == (256, 128, 32)


@pytest.mark.parametrize("bad,why", [
    ({"ffn.0": "shape"}, "packed 256 -> 128"),
    ({"ffn.0": "missing"}, "no such submodule"),
    ({"ffn.0": "gelu"}, "not an nn.Linear"),
    ({"ffn.0": "bias"}, "bias missing"),
    ({"ffn.0": "type"}, "the packed layer is"),
])
def test_a_bad_target_in_the_middle_swaps_nothing(bad, why):
    m = Block()
    before = {n: id(c) for n, c in m.named_modules()}
    targets = {"q": _packed(256, 128, 32), "o": _packed(128, 256, 0, bias=False),
               "ffn.0": _packed(256, 384, 16), "ffn.2": _packed(384, 256, 32)}
    kind = bad["ffn.0"]
    if kind == "shape":
        targets["ffn.0"] = _packed(256, 128, 16)
    elif kind == "missing":
        targets["ffn.7"] = targets.pop("ffn.0")
    elif kind == "gelu":
        targets["ffn.1"] = targets.pop("ffn.0")
    elif kind == "bias":
        targets["ffn.0"] = _packed(256, 384, 16, bias=False)
    else:
        targets["ffn.0"] = np.zeros(3)
    with pytest.raises(InstallError, match=why) as ei:
        install(m, targets)
    assert len(ei.value.problems) == 1
    # nothing was swapped, the good targets before and after the bad one included
    assert {n: id(c) for n, c in m.named_modules()} == before
    assert all(isinstance(c, (torch.nn.Linear, torch.nn.GELU, torch.nn.Sequential, Block))
               for c in m.modules())


def test_every_problem_is_listed():
    m = Block()
    with pytest.raises(InstallError) as ei:
        install(m, {"q": _packed(256, 64, 32), "nope": _packed(256, 128, 0),
                    "o": _packed(128, 256, 0, bias=True)})
    assert len(ei.value.problems) == 3


# ----------------------------------------------- checks before any launch


@pytest.fixture(scope="module")
def layer():
    return _packed(256, 64, 32)


@pytest.mark.parametrize("case", ["wrong K", "3-D x", "fp16 x", "y shape", "y dtype",
                                  "y_dtype name", "ws dtype", "ws small"])
def test_forward_rejects_bad_arguments_before_launch(layer, case):
    M = 4
    x = torch.zeros((M, 256), dtype=torch.float32)
    kw = {}
    if case == "wrong K":
        x = torch.zeros((M, 128))
    elif case == "3-D x":
        x = torch.zeros((1, M, 256))
    elif case == "fp16 x":
        x = x.half()
    elif case == "y shape":
        kw["y"] = torch.empty((M, 65))
    elif case == "y dtype":
        kw["y"] = torch.empty((M, 64), dtype=torch.bfloat16)   # y_dtype 'f32' by default
    elif case == "y_dtype name":
        kw["y_dtype"] = "f16"
    elif case == "ws dtype":
        kw["workspace"] = torch.empty(1 << 16, dtype=torch.int32)
    elif case == "ws small":
        kw["workspace"] = torch.empty(16, dtype=torch.uint8)
    with pytest.raises((ValueError, TypeError)):
        layer.forward(x, **kw)


def test_group_rejects_mixed_shapes(layer):
    from wam_asp_w4a4_amd.layer import forward_group
    other = _packed(384, 64, 32)
    with pytest.raises(ValueError, match="one K"):
        forward_group([layer, other], torch.zeros((2, 256)))
    with pytest.raises(ValueError):
        forward_group([layer, layer], torch.zeros((2, 256)), ys=[torch.empty((2, 64))])
