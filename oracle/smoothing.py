"""Per-layer smoothing search, as plain float64 NumPy steps.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Model card "FastWAM UR3 3-task -- 4-bit quantisations", section "What ASP is,
and what the deflated form means": the smoothing of each layer is not fixed;
its exponents (alpha, beta) are picked from a grid of candidates, following
SVDQuant's protocol, by the error of that layer's own deflated-ASP NVFP4 output
on calibration activations.

Readings taken where the page is silent or loose:

* Smoothing vector of a candidate: s_k = max_m |x_mk|^alpha / max_n |W_nk|^beta,
  computed in float64 and rounded to float32 (the fixed-alpha workloads use the
  same form with alpha = beta = 0.5); a zero column maximum is replaced by 1e-5.
* The grid: alpha runs over 0, 0.05, ..., 0.95 and beta is 0 or 1 - alpha.  That
  literal product has 40 pairs while the page counts 39; the pair alpha = 0,
  beta = 1 (weight-side scaling with no activation smoothing at all) is the one
  left out, which keeps alpha = beta = 0 (no smoothing) as the baseline.
* The error: mean over the M x N outputs of the squared difference between the
  quantised layer (``asp.forward``) and the unquantised x W^T + b.
* Ties: the earlier candidate in the grid order below wins.
"""

import numpy as np

from . import asp


def grid():
    """The 39 (alpha, beta) candidates, beta = 0 first for every alpha, then beta = 1 - alpha."""
    alphas = [i / 20.0 for i in range(20)]
    return [(a, 0.0) for a in alphas] + [(a, 1.0 - a) for a in alphas if a > 0.0]


def smoothing_vector(x_colmax, w_colmax, alpha, beta):
    """float32 s from the column maxima of |x| and |W| (float64 arithmetic)."""
    xm = np.where(np.asarray(x_colmax, np.float64) > 0.0, np.asarray(x_colmax, np.float64), 1e-5)
    wm = np.where(np.asarray(w_colmax, np.float64) > 0.0, np.asarray(w_colmax, np.float64), 1e-5)
    return (xm ** alpha / wm ** beta).astype(np.float32)


def search(x, w, bias, v, candidates):
    """Mean squared output error of every candidate and the index of the smallest."""
    x64 = np.asarray(x, np.float64)
    w64 = np.asarray(w, np.float64)
    ref = x64 @ w64.T
    if bias is not None:
        ref = ref + np.asarray(bias, np.float64)[None, :]
    xmax = np.abs(x64).max(axis=0)
    wmax = np.abs(w64).max(axis=0)
    mse = np.empty(len(candidates))
    for i, (a, b) in enumerate(candidates):
        s = smoothing_vector(xmax, wmax, a, b)
        y = asp.forward(x, w, bias, s, v)
        mse[i] = np.mean((y - ref) ** 2)
    return mse, int(np.argmin(mse))
