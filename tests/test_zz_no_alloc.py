"""asp_forward_noalloc (the workspace in the library's own device array)
against asp_forward (the caller's workspace), through the C ABI: the same
kernels, so the same bits; two calls in a row, the second smaller, then
one whose workspace exceeds the array (rejected before anything runs)."""

import numpy as np
import pytest
import torch

from wam_asp_w4a4_amd import binding as B
from wam_asp_w4a4_amd import synth
from wam_asp_w4a4_amd.layer import PackedLayer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _x(lay):
    if lay.x_dtype == "bf16":
        return torch.from_numpy(synth.bf16_bits(lay.x)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(lay.x)).to(DEV)


def _noalloc(p, x, y_dtype):
    M = x.shape[0]
    y = torch.empty((M, p.N), dtype=torch.float32 if y_dtype == "f32" else torch.bfloat16,
                    device=DEV)
    B.asp_forward_noalloc(x, B.ASP_BF16 if x.dtype == torch.bfloat16 else B.ASP_F32, M, p.N,
                          p.K, p.r, p.prep, p.w_codes, p.w_scales, p.wv, p.bias, y,
                          B.DTYPES[y_dtype])
    return y


def test_noalloc_equals_forward_on_two_calls():
    big = synth.workload(3)[0]                          # 4096 x 3072 -> 3072, r = 32
    small = synth.make_layer("small", 77, 384, 200, 24, seed=3, dtype="f32")
    for lay in (big, small):
        print(f"noalloc {lay.name} M={lay.M} K={lay.K} N={lay.N} r={lay.r}", flush=True)
        p = PackedLayer.pack(lay.w, lay.s, lay.v, lay.b, DEV)
        x = _x(lay)
        for y_dtype in ("f32", "bf16"):
            want = p.forward(x, y_dtype)
            got = _noalloc(p, x, y_dtype)
            torch.cuda.synchronize()
            assert torch.equal(got, want), (lay.name, y_dtype)


def test_noalloc_rejects_a_workspace_above_the_array():
    # 8192 x 14336 activations need 66 MB of codes and scales: above 48 MiB
    M, K, N = 8192, 14336, 16
    need = B.asp_workspace_bytes(M, N, K, 0)
    assert need > (48 << 20)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    dummy = torch.empty(256, dtype=torch.uint8, device=DEV)
    with pytest.raises(B.ASPError) as ei:
        B.asp_forward_noalloc(dummy, B.ASP_BF16, M, N, K, 0, dummy, dummy, dummy, None, None, y,
                              B.DTYPES["f32"])
    assert ei.value.status == 5 and "allocation-free" in str(ei.value)
