"""Pins for the oracle's SVDQuant-style INT4 W4A4 layer (CPU only).

Model card "FastWAM UR3 3-task -- 4-bit quantisations": method table (INT4,
group 64, W4A4, INT8 tensor cores, 4.5798 bits per weight) and section
"Verification -- INT4 SVDQuant".

What pins what:
* hand-worked groups (``tests/golden/int4_groups.txt``): the bfloat16 scale,
  ties to even, and a value whose code depends on the scale being rounded;
* quantiser properties: round-trip error within half a scale step, sign
  symmetry, power-of-two equivariance, code range;
* the rank-r branch: a weight of exact rank r leaves a zero residual and zero
  codes; the residual is orthogonal to the branch; no other rank-r projection
  leaves a smaller residual (Eckart-Young);
* the quantisation-off identity y = x W^T + b (smoothing cancels, branch plus
  residual is the whole weight);
* brute force of the group contraction with Python integers;
* the bits per weight the reading implies for the 600-layer set against the
  model card's 4.5798 (16-bit group scales; 32-bit ones would not fit).
"""

import os

import numpy as np
import pytest

from oracle import svdquant as SQ
from wam_asp_w4a4_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_groups():
    out = []
    for line in open(os.path.join(GOLDEN, "int4_groups.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, ent, scale, codes = [p.strip() for p in line.split("|")]
        v = np.zeros(64, np.float32)
        for tok in ent.split():
            i, val = tok.split(":")
            v[int(i)] = np.float32(float(val))
        c = np.zeros(64, np.int8)
        for tok in codes.split():
            i, val = tok.split(":")
            c[int(i)] = int(val)
        out.append((name, v, float(scale), c))
    return out


@pytest.mark.parametrize("name,v,scale,codes", _golden_groups())
def test_golden_groups(name, v, scale, codes):
    c, s = SQ.quantize_int4(v[None, :])
    assert s[0, 0] == scale, name
    np.testing.assert_array_equal(c[0], codes, err_msg=name)


def test_quantizer_properties():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal((50, 256)) * np.exp(rng.uniform(-8, 8, (50, 1)))).astype(np.float32)
    c, s = SQ.quantize_int4(v)
    assert c.min() >= -8 and c.max() <= 7
    deq = SQ.dequantize_int4(c, s)
    step = np.repeat(s, 64, axis=1)
    # |v / scale| <= 7 (1 + 2^-8) < 7.5, so no value is clamped: error <= half a step
    assert np.all(np.abs(deq - v) <= 0.5 * step * (1 + 1e-6))
    c2, s2 = SQ.quantize_int4(-v)
    np.testing.assert_array_equal(c2, -c)
    np.testing.assert_array_equal(s2, s)
    c3, s3 = SQ.quantize_int4(v * np.float32(2.0 ** 5))
    np.testing.assert_array_equal(c3, c)
    np.testing.assert_array_equal(s3, s * 2.0 ** 5)


def test_exact_rank_weight_leaves_no_residual():
    rng = np.random.default_rng(1)
    N, K, r = 48, 128, 6
    # small-integer factors: the product is exact in float32, so W has rank r exactly
    w = (rng.integers(-4, 5, (N, r)) @ rng.integers(-4, 5, (r, K))).astype(np.float32)
    s = np.exp(rng.uniform(-1, 1, K)).astype(np.float32)
    pk = SQ.pack_weight(w, s, r)
    top = np.abs(pk["w_hat"]).max()
    assert np.abs(pk["resid"]).max() <= 1e-12 * top
    # the residual's codes quantise rounding noise: their values are negligible
    assert np.abs(SQ.dequantize_int4(pk["codes"], pk["scales"])).max() <= 1e-12 * top


def test_branch_is_the_best_rank_r_part():
    rng = np.random.default_rng(2)
    lay = synth.make_svdq_layer("t", 8, 256, 96, 16, seed=3, planted=16)
    pk = SQ.pack_weight(lay.w, lay.s, 16)
    l2, resid = pk["l2"], pk["w_hat"] - pk["l1"] @ pk["l2"]
    np.testing.assert_allclose(l2 @ l2.T, np.eye(16), atol=1e-12)
    idx = np.argmax(np.abs(l2), axis=1)
    assert np.all(l2[np.arange(16), idx] > 0)
    assert np.abs(resid @ l2.T).max() <= 1e-9 * np.abs(pk["w_hat"]).max()
    best = np.linalg.norm(resid)
    for _ in range(20):
        q = np.linalg.qr(rng.standard_normal((256, 16)))[0]
        assert np.linalg.norm(pk["w_hat"] - pk["w_hat"] @ q @ q.T) >= best


def test_quantisation_off_identity():
    lay = synth.make_svdq_layer("t", 16, 256, 64, 32, seed=4)
    y = SQ.forward(lay.x, lay.w, lay.b, lay.s, 32, quantize=False)
    ref = lay.x.astype(np.float64) @ lay.w.astype(np.float64).T + lay.b
    # x_hat is rounded to float32 once and R once: a few float32 ulps of the terms
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) <= 1e-6


def test_quantised_layer_is_close():
    lay = synth.make_svdq_layer("t", 32, 512, 128, 32, seed=5)
    y = SQ.forward(lay.x, lay.w, lay.b, lay.s, 32)
    ref = lay.x.astype(np.float64) @ lay.w.astype(np.float64).T + lay.b
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert 1e-3 < rel < 0.1


def test_group_contraction_brute_force():
    rng = np.random.default_rng(6)
    M, N, K, r = 3, 4, 128, 2
    xc = rng.integers(-8, 8, (M, K)).astype(np.int8)
    wc = rng.integers(-8, 8, (N, K)).astype(np.int8)
    xs = SQ.round_bf16(rng.uniform(0.01, 2, (M, K // 64)))
    ws = SQ.round_bf16(rng.uniform(0.01, 2, (N, K // 64)))
    u = SQ.round_bf16(rng.standard_normal((M, r)))
    l1 = SQ.round_bf16(rng.standard_normal((N, r)))
    b = rng.standard_normal(N)
    y = SQ.output_from_codes(xc, xs, wc, ws, u, l1, b)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for g in range(K // 64):
                isum = sum(int(xc[m, k]) * int(wc[n, k]) for k in range(64 * g, 64 * g + 64))
                acc += isum * float(xs[m, g]) * float(ws[n, g])
            acc += sum(float(u[m, j]) * float(l1[n, j]) for j in range(r)) + b[n]
            assert abs(acc - y[m, n]) <= 1e-12 * max(1.0, abs(acc))


def test_bits_per_weight_against_model_card():
    card = None
    for line in open(os.path.join(GOLDEN, "svdq_bits.txt")):
        if line.startswith("bits_per_weight"):
            card = float(line.split()[1])
    shapes = synth.mot_shapes()
    weights = sum(n * k for _, m, k, n, *_ in shapes)

    def bpw(scale_bits, extra_vectors):
        bits = sum(n * k * 4 + (n * k // SQ.GROUP) * scale_bits + 32 * (n + k) * 16
                   + extra_vectors * 16 * (n + k) for _, m, k, n, *_ in shapes)
        return bits / weights
    # 4-bit codes, a 16-bit scale per 64 weights, a rank-32 bf16 branch on every
    # layer, plus the 16-bit smoothing vector and bias: within 0.01 of the card
    assert abs(bpw(16, 1) - card) < 0.01
    assert abs(bpw(32, 1) - card) > 0.2
