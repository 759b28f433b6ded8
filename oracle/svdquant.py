"""SVDQuant-style INT4 W4A4 linear layer (group 64), in plain NumPy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Model card "FastWAM UR3 3-task -- 4-bit quantisations", the method table (the
second checkpoint: SVDQuant, INT4 with groups of 64 for both weights and
activations, contracted on INT8 tensor cores, which are exact for 4-bit codes;
4.58 bits per weight) and section "Verification -- INT4 SVDQuant" (activation
scales reproduced exactly, at most 0.1 % of codes one step apart).  The layer
follows SVDQuant's decomposition: the smoothed weight W_hat = W diag(s) is split
into a rank-r 16-bit branch L1 L2 (its truncated SVD) and a residual R that is
quantised to 4 bits together with the smoothed activation x_hat = x / s:

    y = x_hat L2^T L1^T + dequant(Q(x_hat) Q(R)^T) + b.

Readings taken where the page is silent (each used identically everywhere):

* smoothing: the same s as the NVFP4 arm (alpha = 0.5), no rotation;
  x_hat = float32(x * float32(1 / s)), one float32 multiply per element;
* quantiser: symmetric, per group of 64 consecutive K elements, scale =
  bfloat16(float32(amax) / 7) (a 16-bit scale, which the 4.58 bits per weight
  imply), code = clamp(round_half_even(float32(v / scale)), -8, 7), a zero
  scale giving zero codes; the division and the rounding are float32, so a
  code is a float32 decision on both sides;
* low-rank branch: L1 L2 is the rank-r truncated SVD of W_hat in float64
  (L2 = the top right singular vectors as rows, each with its largest-magnitude
  entry positive, L1 = W_hat L2^T), stored in bfloat16; R = W_hat - L1 L2
  from the unrounded factors, rounded to float32, then quantised; u = x_hat
  L2^T in float64 then rounded to bfloat16, and the branch is u times
  bfloat16(L1)^T;
* the group products are exact integers; each is scaled by the product of
  its two bfloat16 scales (exact in float32); everything else is float64 here.
"""

import numpy as np

from . import asp as _asp

GROUP = 64


def round_bf16(a):
    """float64 array -> nearest bfloat16 values (ties to even), as float64."""
    return _asp.round_bf16(np.asarray(a, np.float64))


def quantize_int4(v):
    """Rows of float32 values (K a multiple of 64) -> (int8 codes, float64 scales).

    Scales are bfloat16 values; codes lie in [-8, 7]."""
    v = np.asarray(v, np.float32)
    rows, cols = v.shape
    if cols % GROUP:
        raise ValueError("K must be a multiple of 64")
    g = v.reshape(rows, cols // GROUP, GROUP)
    amax = np.abs(g).max(axis=2).astype(np.float32)
    scale = round_bf16(amax / np.float32(7.0))              # float32 quotient, then bf16
    s32 = scale.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s32[..., None] > 0, g / s32[..., None], np.float32(0.0)).astype(np.float32)
    codes = np.clip(np.rint(q), -8, 7).astype(np.int8)    # rint: half to even
    return codes.reshape(rows, cols), scale


def dequantize_int4(codes, scales):
    c = np.asarray(codes, np.float64)
    rows, cols = c.shape
    return (c.reshape(rows, cols // GROUP, GROUP) * np.asarray(scales, np.float64)[..., None]).reshape(rows, cols)


def smoothed_activation(x, s):
    """x_hat = float32(x * float32(1 / s))."""
    rs = (1.0 / np.asarray(s, np.float64)).astype(np.float32)
    return (np.asarray(x, np.float32) * rs[None, :]).astype(np.float32)


def low_rank(w_hat, r):
    """(L1 N x r, L2 r x K) of the rank-r truncated SVD of w_hat, float64; each
    row of L2 (a right singular vector) has its largest-magnitude entry positive."""
    _, _, vt = np.linalg.svd(np.asarray(w_hat, np.float64), full_matrices=False)
    l2 = vt[:r].copy()
    idx = np.argmax(np.abs(l2), axis=1)
    l2 *= np.where(l2[np.arange(r), idx] < 0, -1.0, 1.0)[:, None]
    return np.asarray(w_hat, np.float64) @ l2.T, l2


def pack_weight(w, s, r):
    """Weight side: W_hat = W diag(s), its rank-r branch and the INT4 residual."""
    w_hat = np.asarray(w, np.float64) * np.asarray(s, np.float64)[None, :]
    l1, l2 = low_rank(w_hat, r) if r > 0 else (np.zeros((w_hat.shape[0], 0)), np.zeros((0, w_hat.shape[1])))
    resid = (w_hat - l1 @ l2).astype(np.float32)
    codes, scales = quantize_int4(resid)
    return {"w_hat": w_hat, "l1": l1, "l2": l2, "resid": resid, "codes": codes, "scales": scales,
            "l1_bf16": round_bf16(l1), "l2": l2}


def activation_side(x, s, l2):
    """(x_hat float32, codes, scales, u as bfloat16 values)."""
    xh = smoothed_activation(x, s)
    codes, scales = quantize_int4(xh)
    u = round_bf16(xh.astype(np.float64) @ np.asarray(l2, np.float64).T)
    return xh, codes, scales, u


def output_from_codes(xc, xs, wc, ws, u, l1_bf16, bias):
    """y from the two sides' codes and scales: exact group products times the
    product of their scales, plus the bfloat16 low-rank branch and the bias."""
    xc = np.asarray(xc, np.int64)
    wc = np.asarray(wc, np.int64)
    M, K = xc.shape
    N = wc.shape[0]
    G = K // GROUP
    y = np.zeros((M, N))
    for g in range(G):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        prod = (xc[:, sl] @ wc[:, sl].T).astype(np.float64)   # exact integers
        y += prod * (np.asarray(xs, np.float64)[:, g:g + 1] * np.asarray(ws, np.float64)[None, :, g])
    if u.shape[1]:
        y += np.asarray(u, np.float64) @ np.asarray(l1_bf16, np.float64).T
    if bias is not None:
        y += np.asarray(bias, np.float64)[None, :]
    return y


def forward(x, w, bias, s, r, packed=None, quantize=True):
    """The whole layer in float64; quantize=False gives x_hat W_hat^T + b."""
    pk = packed if packed is not None else pack_weight(w, s, r)
    xh, xc, xs, u = activation_side(x, s, pk["l2"])
    if not quantize:
        y = xh.astype(np.float64) @ (pk["l1"] @ pk["l2"] + pk["resid"].astype(np.float64)).T
        return y + (0.0 if bias is None else np.asarray(bias, np.float64)[None, :])
    return output_from_codes(xc, xs, pk["codes"], pk["scales"], u, pk["l1_bf16"], bias)
