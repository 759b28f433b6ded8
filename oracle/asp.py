"""The deflated ASP NVFP4 W4A4 linear layer, as plain float64 NumPy steps.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Model card "FastWAM UR3 3-task -- 4-bit quantisations", section "What ASP is,
and what the deflated form means": with s the smoothing vector, H a block
Hadamard, V the rank-32 basis and W_tilde the smoothed weight,

    x_tilde = (x / s) H
    y = (x_tilde V)(W_tilde V)^T + NVFP4GEMM((I - V V^T) x_tilde, W_tilde (I - V V^T)) + bias

"Deflated" means the protected subspace is removed from the 4-bit path on both
sides; the low-rank branch holds the exact W_tilde V and stays in bf16.  The
same page's verification section puts its per-layer error down to rounding the
output to bf16.  The Q-WAM abstract describes the same split: a 16-bit low-rank
branch plus the 4-bit complement of weights and activations.

Readings taken where the page is silent or loose (row-vector convention,
x: M x K, W: N x K, y = x W^T + b):

* W_tilde includes the rotation: W_tilde = W diag(s) H.  Only then does the
  unquantised contract reproduce x W^T + b, because the activation is rotated.
* (I - V V^T) x_tilde is read as the row form x_tilde - (x_tilde V) V^T.
* The deflated operands are rounded to float32 before NVFP4 quantisation (the
  quantiser is defined on float32 rows); V, s, W, x, b are float32 inputs.
* The low-rank branch multiplies bf16(u) by bf16(W_tilde V), u = x_tilde V; the
  deflation itself uses the unrounded u.
* Everything else is float64; the result y is float64 (a bf16-output device
  path is compared against it without re-rounding).

``quantize=False`` replaces NVFP4 quantise/dequantise and the bf16 roundings
by the identity; then y equals x W^T + b up to float64 rounding.

The same section mentions a cheaper shared-weight arm that keeps a single 4-bit
weight with only the basis V beside it (``form="shared"``).  Reading taken:
the 4-bit weight is W_tilde itself, not deflated, and the low-rank factor is derived from that one
quantised weight, L = DQ(Q(W_tilde)) V.  The activation side is the same.
Without quantisation it also gives x W^T + b: (x_tilde V)(W_tilde V)^T +
(x_tilde - x_tilde V V^T) W_tilde^T = x_tilde W_tilde^T, the projector being
needed on one side only.
"""

import numpy as np

from . import formats
from .hadamard import block_rotate, HADAMARD_BLOCK


def round_to_precision(x, p: int, emin: int):
    """Round float64 values to a binary float format with p significant bits.

    Round to nearest, ties to even; ``emin`` is the exponent of the smallest
    normal number (values below it share its quantum, i.e. gradual underflow).
    No overflow handling (the values rounded here are far from any format max).
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    lead = np.maximum(e - 1, emin)
    quantum = np.ldexp(1.0, lead - (p - 1))
    return np.rint(x / quantum) * quantum


def round_bf16(x):
    """float64 -> nearest bfloat16 value (8 significant bits, RNE), as float64."""
    return round_to_precision(x, 8, -126)


def round_fp32(x):
    """float64 -> nearest float32 (IEEE conversion, RNE)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def _basis(v, k):
    if v is None:
        return np.zeros((k, 0), dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if v.shape[0] != k:
        raise ValueError("V must be K x r")
    return v


def pack_weight(w, s, v=None, block: int = HADAMARD_BLOCK, form: str = "deflated"):
    """Weight side, done once per layer.

    Deflated arm: W_tilde = W diag(s) H;  L = W_tilde V;  W_d = W_tilde - L V^T;
    NVFP4(float32(W_d)) row-wise along K;  L kept as bf16.
    Shared arm: NVFP4(float32(W_tilde));  L = DQ(that) V, kept as bf16.
    Returns a dict with the codes, scales, bf16 low-rank factor (float64 array
    holding bf16 values, N x r) and the intermediates; "w_4bit" and "low_rank"
    are the unquantised weight of the 4-bit path and low-rank factor.
    """
    if form not in ("deflated", "shared"):
        raise ValueError(f"unknown weight form {form!r}")
    w = np.asarray(w, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    n, k = w.shape
    vb = _basis(v, k)
    w_tilde = block_rotate(w * s[None, :], block)
    if form == "deflated":
        low_rank = w_tilde @ vb
        w_4bit = w_tilde - low_rank @ vb.T
        w_pre = round_fp32(w_4bit)
        codes, scales = formats.quantize_nvfp4(w_pre)
        lr_stored = low_rank
    else:
        low_rank = w_tilde @ vb
        w_4bit = w_tilde
        w_pre = round_fp32(w_4bit)
        codes, scales = formats.quantize_nvfp4(w_pre)
        lr_stored = formats.dequantize_nvfp4(codes, scales) @ vb
    return {
        "w_codes": codes,
        "w_scales": scales,
        "wv": round_bf16(lr_stored),
        "w_prequant": w_pre,
        "w_tilde": w_tilde,
        "w_4bit": w_4bit,
        "w_deflated": w_tilde - low_rank @ vb.T,
        "low_rank": low_rank,
    }


def activation_side(x, s, v=None, block: int = HADAMARD_BLOCK):
    """Activation side, done on every call.

    x_tilde = (x / s) H;  u = x_tilde V;  x_d = x_tilde - u V^T;
    NVFP4(float32(x_d)) row-wise along K.
    """
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    _, k = x.shape
    vb = _basis(v, k)
    x_tilde = block_rotate(x / s[None, :], block)
    u = x_tilde @ vb
    x_defl = x_tilde - u @ vb.T
    x_pre = round_fp32(x_defl)
    codes, scales = formats.quantize_nvfp4(x_pre)
    return {
        "x_codes": codes,
        "x_scales": scales,
        "u": u,
        "x_prequant": x_pre,
        "x_tilde": x_tilde,
        "x_deflated": x_defl,
    }


def output_from_codes(x_codes, x_scales, u, w_codes, w_scales, wv, bias=None):
    """The contraction given both operands' NVFP4 codes and the low-rank inputs.

    y = DQ(x) DQ(W)^T + bf16(u) wv^T + b, all in float64.  ``wv`` holds bf16
    values already; ``u`` is rounded to bf16 here.
    """
    xa = formats.dequantize_nvfp4(x_codes, x_scales)
    wa = formats.dequantize_nvfp4(w_codes, w_scales)
    y = xa @ wa.T
    u = np.asarray(u, dtype=np.float64)
    if u.shape[1]:
        y = y + round_bf16(u) @ np.asarray(wv, dtype=np.float64).T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def forward(x, w, bias, s, v=None, quantize: bool = True, packed=None,
            block: int = HADAMARD_BLOCK, form: str = "deflated"):
    """y (float64, M x N) of the ASP linear (deflated or shared-weight arm) for
    the inputs given.

    ``packed`` may hold an earlier ``pack_weight`` result for the same (w, s, v, form).
    """
    if packed is None:
        packed = pack_weight(w, s, v, block, form)
    act = activation_side(x, s, v, block)
    if not quantize:
        y = act["x_deflated"] @ packed["w_4bit"].T + act["u"] @ packed["low_rank"].T
        if bias is not None:
            y = y + np.asarray(bias, dtype=np.float64)[None, :]
        return y
    return output_from_codes(act["x_codes"], act["x_scales"], act["u"],
                             packed["w_codes"], packed["w_scales"], packed["wv"], bias)
