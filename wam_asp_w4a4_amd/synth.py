"""Seeded synthetic layer inputs shaped like a two-expert MoT's quantised linears.

This module only draws inputs (activations, weights, bias, basis, smoothing
vector); it holds none of the layer's arithmetic, and both the device path and
the CPU oracle's tests consume what it returns.  The trained weights and the
calibration data the model card "FastWAM UR3 3-task -- 4-bit quantisations"
refers to are not available, so these seeded draws stand in for them with the
layer shapes that page lists (two experts x 30 blocks x {self_attn q/k/v/o,
cross_attn q/k/v/o, ffn.0, ffn.2}) and the Q-WAM paper's action-expert-only
protection (rank 32 on the action expert, plain smoothed+rotated NVFP4 on the
video expert).

Recipe, per layer (NumPy PCG64 ``default_rng(seed)``, fixed draw order):
  1. x ~ N(0, 1), shape M x K (or GELU(N(0,1)) for an ffn.2 input);
  2. n = round(p * K) outlier channels drawn without replacement; those whole
     columns are multiplied by ``outlier_gain``;
  3. W ~ N(0, 1/K) (standard deviation 1/sqrt(K)), shape N x K;
  4. b ~ N(0, 0.01) (standard deviation 0.1), length N;
  5. G ~ N(0, 1), K x r; V = Q of the reduced QR of G (orthonormal columns);
  x and W are then rounded to bf16 when the layer's dtype is bf16 (the arrays
  stay float32, holding bf16-exact values);
  s_k = max_m |x_mk|^alpha / max_n |W_nk|^(1 - alpha) from the rounded x and W
  in float64 (a zero maximum is replaced by 1e-5), then rounded to float32.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

try:  # exact float32 -> bfloat16 RNE rounding; torch is part of the runtime
    import torch
except Exception:  # pragma: no cover
    torch = None

DEFAULT_SEED = 42


def to_bf16_values(a: np.ndarray) -> np.ndarray:
    """Round a float32 array to the nearest bfloat16 values (RNE); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if torch is not None:
        return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    bits = a.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of a float32 array that holds bf16-exact values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("array holds values that are not bf16-exact")
    return (bits >> 16).astype(np.uint16)


@dataclass
class Layer:
    name: str
    M: int
    K: int
    N: int
    r: int
    x: np.ndarray          # M x K float32 (bf16-exact when x_dtype == "bf16")
    x_dtype: str           # "f32" or "bf16"
    w: np.ndarray          # N x K float32
    b: np.ndarray          # N float32
    s: np.ndarray          # K float32
    v: np.ndarray | None   # K x r float32, orthonormal columns; None when r == 0
    meta: dict = field(default_factory=dict)


def _gelu(z: np.ndarray) -> np.ndarray:
    """Exact (erf) GELU of the standard-normal draws."""
    from scipy.special import erf
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def smoothing_vector(x: np.ndarray, w: np.ndarray, alpha: float = 0.5) -> np.ndarray:
    ax = np.abs(x.astype(np.float64)).max(axis=0) if x.shape[0] else np.zeros(x.shape[1])
    aw = np.abs(w.astype(np.float64)).max(axis=0) if w.shape[0] else np.zeros(w.shape[1])
    ax = np.where(ax > 0, ax, 1e-5)
    aw = np.where(aw > 0, aw, 1e-5)
    return (ax ** alpha / aw ** (1.0 - alpha)).astype(np.float32)


def draw_activation(rng, M, K, outlier_frac, outlier_gain, gelu=False):
    z = rng.standard_normal((M, K))
    x = _gelu(z) if gelu else z
    n_out = int(round(outlier_frac * K))
    idx = np.sort(rng.choice(K, size=n_out, replace=False)) if n_out else np.zeros(0, int)
    x[:, idx] *= outlier_gain
    return x, idx


def draw_basis(rng, K, r):
    if r == 0:
        return None
    g = rng.standard_normal((K, r))
    q, _ = np.linalg.qr(g)
    return q.astype(np.float32)


def make_svdq_layer(name, M, K, N, r, *, seed=DEFAULT_SEED, dtype="bf16", outlier_frac=0.01,
                    outlier_gain=20.0, planted=32, alpha=0.5) -> Layer:
    """A seeded layer for the SVDQuant-style arm: the weight carries a planted
    low-rank part above its N(0, 1/K) bulk, the structure that arm's 16-bit
    branch is meant to take (after smoothing, a trained weight's leading
    singular values stand out from the rest).

    Draw order (PCG64 ``default_rng(seed)``): x as ``draw_activation``; the bulk
    W0 ~ N(0, 1/K); b ~ N(0, 0.01); U (N x planted) and Q (K x planted) from
    the QR of N(0, 1) draws; W = W0 + U diag(sig) Q^T with
    sig = (1 + sqrt(N / K)) * linspace(8, 4, planted), i.e. 8 to 4 times the
    bulk's largest singular value; then x and W are rounded to bf16 and s is
    drawn from them as for the other layers.  ``r`` is the rank the layer is
    packed with.
    """
    rng = np.random.default_rng(seed)
    x64, idx = draw_activation(rng, M, K, outlier_frac, outlier_gain)
    x32 = x64.astype(np.float32)
    w0 = rng.standard_normal((N, K)) / math.sqrt(K)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    u, _ = np.linalg.qr(rng.standard_normal((N, planted)))
    q, _ = np.linalg.qr(rng.standard_normal((K, planted)))
    sig = (1.0 + math.sqrt(N / K)) * np.linspace(8.0, 4.0, planted)
    w = (w0 + (u * sig) @ q.T).astype(np.float32)
    if dtype == "bf16":
        x32 = to_bf16_values(x32)
        w = to_bf16_values(w)
    s = smoothing_vector(x32, w, alpha)
    return Layer(name, M, K, N, r, x32, dtype, w, b, s, None,
                 {"seed": seed, "outlier_channels": idx, "planted": planted})


def draw_metric(rng, K, decay=8.0, floor=1e-6, rank=None):
    """Synthetic symmetric PSD K x K metric with a fast-falling spectrum.

    Stands in for a layer's action metric (an expectation of J^T J, which needs
    the trained model): Q = orthogonal factor of the QR of a K x K N(0, 1) draw,
    lam_i = exp(-i / decay) + floor for i < rank (rank = K by default) and 0
    beyond, G = Q diag(lam) Q^T in float64, made exactly symmetric and rounded
    to float32.  Returns (G float32, lam float64 descending, Q float64).
    """
    rank = K if rank is None else rank
    q, _ = np.linalg.qr(rng.standard_normal((K, K)))
    i = np.arange(K, dtype=np.float64)
    lam = np.where(i < rank, np.exp(-i / decay) + floor, 0.0)
    g = (q * lam) @ q.T
    g = 0.5 * (g + g.T)
    return g.astype(np.float32), lam, q


def draw_metric_reflected(rng, K, r, n_reflections=4, decay=8.0, floor=1e-6):
    """A large synthetic metric with a known spectrum and known leading
    eigenvectors, without a dense K x K orthogonal draw: Q = H_1 ... H_n, a
    product of Householder reflections H = I - 2 u u^T (u random, unit), and
    G = Q diag(lam) Q^T with lam_i = exp(-i / decay) + floor, built in float64
    by applying the reflections to diag(lam) (O(n K^2)), made exactly
    symmetric and rounded to float32.  Returns (G float32, lam float64
    descending, the first r columns of Q float64)."""
    lam = np.exp(-np.arange(K, dtype=np.float64) / decay) + floor
    us = []
    for _ in range(n_reflections):
        u = rng.standard_normal(K)
        us.append(u / np.linalg.norm(u))
    g = np.diag(lam)
    # G = H_1 (H_2 (... diag(lam) ...) H_2) H_1: innermost reflection first
    for u in reversed(us):
        gu = g @ u
        ugu = u @ gu
        g -= 2.0 * np.outer(u, gu)
        g -= 2.0 * np.outer(gu, u)
        g += 4.0 * ugu * np.outer(u, u)
    g = 0.5 * (g + g.T)
    q = np.eye(K, r)
    for u in reversed(us):
        q -= 2.0 * np.outer(u, u @ q)
    return g.astype(np.float32), lam, q


def draw_start(rng, K, p):
    """K x p float32 N(0, 1) starting block for a subspace iteration."""
    return rng.standard_normal((K, p)).astype(np.float32)


def make_layer(name, M, K, N, r, *, seed=DEFAULT_SEED, dtype="bf16",
               outlier_frac=0.01, outlier_gain=20.0, gelu=False, alpha=0.5,
               x=None, v=None) -> Layer:
    """One seeded layer.  ``x`` / ``v`` may be passed in to share them between layers."""
    rng = np.random.default_rng(seed)
    if x is None:
        x64, idx = draw_activation(rng, M, K, outlier_frac, outlier_gain, gelu)
        x32 = x64.astype(np.float32)
        if dtype == "bf16":
            x32 = to_bf16_values(x32)
    else:
        x32, idx = x, None
    w = (rng.standard_normal((N, K)) / math.sqrt(K)).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    if v is None:
        v = draw_basis(rng, K, r)
    if dtype == "bf16":
        w = to_bf16_values(w)
    s = smoothing_vector(x32, w, alpha)
    return Layer(name, M, K, N, r, x32, dtype, w, b, s, v,
                 {"seed": seed, "outlier_channels": idx})


# ---------------------------------------------------------------------------
# The five workloads: 0 = small single layer (oracle in seconds), 1 = action
# attention projection pair, 2 = action FFN pair, 3 = video attention
# projection, 4 = the two-expert layer set (generated layer by layer).
# ---------------------------------------------------------------------------

WORKLOADS = {
    0: "single deflated-ASP linear, M=64 K=N=512 r=32, fp32 x",
    1: "action-expert attention projection pair, M=256 K=N=1024 r=32, bf16",
    2: "action-expert FFN pair, ffn.0 256x1024->4096, ffn.2 256x4096->1024, r=32, bf16",
    3: "video-expert attention projection, M=4096 K=N=3072 r=32, bf16",
    4: "two-expert MoT layer set, 600 linears x 10 denoising steps",
}


def workload(idx: int, seed: int = DEFAULT_SEED) -> list[Layer]:
    if idx == 0:
        return [make_layer("single", 64, 512, 512, 32, seed=seed, dtype="f32")]
    if idx == 1:
        first = make_layer("attn.a", 256, 1024, 1024, 32, seed=seed)
        # the pair shares x and V; each layer draws its own W, b (and so its own s)
        second = make_layer("attn.b", 256, 1024, 1024, 32, seed=seed + 1,
                            x=first.x, v=first.v)
        return [first, second]
    if idx == 2:
        return [make_layer("ffn.0", 256, 1024, 4096, 32, seed=seed),
                make_layer("ffn.2", 256, 4096, 1024, 32, seed=seed + 1, gelu=True)]
    if idx == 3:
        return [make_layer("video.attn", 4096, 3072, 3072, 32, seed=seed,
                           outlier_frac=0.005, outlier_gain=30.0)]
    if idx == 4:
        return list(mot_layer_set(seed))
    raise ValueError(f"unknown workload {idx}")


MOT_EXPERTS = {
    # expert: (d_model, d_ffn, tokens M, rank, outlier fraction, outlier gain)
    "video": (3072, 14336, 4096, 0, 0.005, 30.0),
    "action": (1024, 4096, 256, 32, 0.01, 20.0),
}
MOT_BLOCKS = 30
MOT_PROJ = ["self_attn.q", "self_attn.k", "self_attn.v", "self_attn.o",
            "cross_attn.q", "cross_attn.k", "cross_attn.v", "cross_attn.o",
            "ffn.0", "ffn.2"]


def mot_shapes():
    """(name, M, K, N, r, outlier_frac, outlier_gain, gelu) for the 600 linears."""
    out = []
    for expert in ("video", "action"):
        d, f, m, r, frac, gain = MOT_EXPERTS[expert]
        for blk in range(MOT_BLOCKS):
            for p in MOT_PROJ:
                k, n = (d, f) if p == "ffn.0" else (f, d) if p == "ffn.2" else (d, d)
                out.append((f"{expert}.{blk}.{p}", m, k, n, r, frac, gain, p == "ffn.2"))
    return out


def mot_layer_set(seed: int = DEFAULT_SEED, only=None):
    """Yield the 600 layers (seed + layer index); ``only`` restricts to indices."""
    for i, (name, m, k, n, r, frac, gain, gelu) in enumerate(mot_shapes()):
        if only is not None and i not in only:
            continue
        yield make_layer(name, m, k, n, r, seed=seed + i, outlier_frac=frac,
                         outlier_gain=gain, gelu=gelu)
