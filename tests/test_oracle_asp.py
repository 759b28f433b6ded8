"""Pins for the oracle's deflated ASP layer (CPU only).

Model card "FastWAM UR3 3-task -- 4-bit quantisations", section "What ASP is,
and what the deflated form means" (the deflated contract) and section
"Verification -- NVFP4 deflated ASP" (residency figures, bf16 output cast).

What pins what:
* rounding helpers against torch's bfloat16 conversion, numpy's float32
  conversion and hand-worked ties;
* basis and projector invariants (V^T V = I, P^2 = P, P V = 0, W_d V = 0);
* the quantisation-off identity y = x W^T + b (smoothing and rotation cancel,
  the two deflations recombine) -- a closed form independent of the code path;
* a constructed layer whose rotated operands lie exactly on the NVFP4 grid and
  whose protected channels are unit vectors, where the quantised y is exactly
  x W^T + b;
* the channel-bypass special case (V = unit vectors in rotated coordinates);
* brute force on tiny layers: dense explicit H (closed form), explicit
  projector, Python loops and exact rational quantiser decisions;
* row independence, and the residency sizes the model card prints.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import asp as A
from oracle import formats as F
from oracle import hadamard as Hd
from wam_asp_w4a4_amd import synth

# ------------------------------------------------------------ rounding helpers


def test_round_bf16_matches_torch_on_float32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(A.round_bf16(x.astype(np.float64)), want)


def test_round_bf16_hand_ties():
    one = 1.0
    assert A.round_bf16(one + 2.0 ** -8) == 1.0                    # tie -> even
    assert A.round_bf16(one + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6    # tie -> even
    assert A.round_bf16(one + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert A.round_bf16(-3.0) == -3.0


def test_round_to_precision_matches_float32_conversion():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000) * np.exp(rng.uniform(-100, 80, 20000))
    x = np.concatenate([x, [0.0, -0.0, 1e-42, -3e-40, 2.0 ** -149 * 1.5]])
    assert np.array_equal(A.round_to_precision(x, 24, -126),
                          x.astype(np.float32).astype(np.float64))


# ----------------------------------------------------------------- invariants


@pytest.fixture(scope="module")
def layer0():
    return synth.workload(0)[0]


def test_basis_and_projector(layer0):
    v = layer0.v.astype(np.float64)
    k, r = v.shape
    assert np.abs(v.T @ v - np.eye(r)).max() < 1e-6  # float32 basis
    p = np.eye(k) - v @ np.linalg.solve(v.T @ v, v.T)  # exact projector of span(V)
    assert np.abs(p @ p - p).max() < 1e-12
    assert np.abs(p - p.T).max() < 1e-12
    assert np.abs(p @ v).max() < 1e-12
    assert abs(np.trace(p) - (k - r)) < 1e-9


def test_weight_deflation_annihilates_basis(layer0):
    pk = A.pack_weight(layer0.w, layer0.s, layer0.v)
    v = layer0.v.astype(np.float64)
    # W_d V = W_tilde V (I - V^T V) vanishes up to V's float32 orthonormality
    scale = np.abs(pk["w_tilde"]).max()
    assert np.abs(pk["w_deflated"] @ v).max() < 1e-5 * scale
    assert pk["w_codes"].shape == (layer0.N, layer0.K // 2)
    assert pk["w_scales"].shape == (layer0.N, layer0.K // 16)
    assert pk["wv"].shape == (layer0.N, layer0.r)


def _orthonormal(v):
    q, _ = np.linalg.qr(np.asarray(v, dtype=np.float64))
    return q


@pytest.mark.parametrize("rank", [0, 32])
def test_quantization_off_identity(layer0, rank):
    # Use an exactly orthonormal float64 basis so the identity holds to fp64 rounding.
    v = _orthonormal(layer0.v)[:, :rank] if rank else None
    y = A.forward(layer0.x, layer0.w, layer0.b, layer0.s, v, quantize=False)
    ref = layer0.x.astype(np.float64) @ layer0.w.astype(np.float64).T + layer0.b
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 1e-12


def test_quantized_output_is_close_but_not_exact(layer0):
    y = A.forward(layer0.x, layer0.w, layer0.b, layer0.s, layer0.v)
    ref = layer0.x.astype(np.float64) @ layer0.w.astype(np.float64).T + layer0.b
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert 1e-3 < rel < 0.2, rel


def test_row_independence(layer0):
    rows = [5, 0, 63, 17]
    full = A.forward(layer0.x, layer0.w, layer0.b, layer0.s, layer0.v)
    part = A.forward(layer0.x[rows], layer0.w, layer0.b, layer0.s, layer0.v)
    assert np.array_equal(full[rows], part)


# --------------------------------------------- constructed exact-output layer


def _grid_matrix(rng, rows, cols, scale_exp):
    """Rows whose 16-blocks are each 2^e x E2M1 values with a 6 in every block."""
    mags = rng.choice(F.E2M1_VALUES[:8], size=(rows, cols))
    signs = rng.choice([-1.0, 1.0], size=(rows, cols))
    a = mags * signs
    a[:, ::16] = 6.0  # block amax = 6 exactly -> scale = 2^e exactly
    e = rng.integers(-scale_exp, scale_exp + 1, size=(rows, cols // 16))
    return a * np.repeat(2.0 ** e, 16, axis=1)


def test_lossless_on_grid_with_unit_basis():
    rng = np.random.default_rng(11)
    m, k, n = 6, 256, 32
    protected = [3, 130]  # channels (in rotated coordinates) held by the bf16 branch
    xh = _grid_matrix(rng, m, k, 3)
    wh = _grid_matrix(rng, n, k, 3)
    # the protected channels hold small bf16-exact values that never set a block max
    xh[:, protected] = rng.choice([0.5, -1.0, 1.5], size=(m, 2))
    wh[:, protected] = rng.choice([0.25, -0.75, 1.0], size=(n, 2))
    v = np.zeros((k, 2))
    v[protected, [0, 1]] = 1.0
    s = np.ones(k)
    h = np.kron(np.eye(k // 128), Hd.sylvester(128)) / np.sqrt(128)
    x = xh @ h     # so that (x / s) H = xh
    w = wh @ h     # so that W diag(s) H = wh
    b = rng.standard_normal(n)
    y = A.forward(x, w, b, s, v)
    # quantisation is lossless, the bf16 branch is exact, so y = xh wh^T + b = x W^T + b
    assert np.abs(y - (xh @ wh.T + b)).max() < 1e-9
    act = A.activation_side(x, s, v)
    assert np.all(act["x_prequant"][:, protected] == 0.0)
    assert np.abs(act["u"] - xh[:, protected]).max() < 1e-12


# ------------------------------------------------------------ brute force


def _bf_quant_block(vals):
    """Exact NVFP4 of 16 float32 values by enumeration in rational arithmetic."""
    e4 = [Fraction(float(c)) for c in F.E4M3_VALUES[:0x7F]]
    e2 = [Fraction(float(c)) for c in F.E2M1_VALUES[:8]]

    def nearest(grid, q):
        best = 0
        for i in range(len(grid)):
            d, db = abs(q - grid[i]), abs(q - grid[best])
            if d < db or (d == db and i % 2 == 0):
                best = i
        return best

    amax = max(abs(Fraction(float(v))) for v in vals)
    q = amax / 6
    sc = 0x7E if q > 448 else nearest(e4, q)
    out = []
    for v in vals:
        mag = 0 if e4[sc] == 0 else (7 if abs(Fraction(float(v))) / e4[sc] > 6
                                     else nearest(e2, abs(Fraction(float(v))) / e4[sc]))
        out.append(float(e2[mag] * e4[sc]) * (-1.0 if np.signbit(v) else 1.0))
    return out


def _bf_forward(x, w, b, s, v, shared=False):
    m, k = x.shape
    n = w.shape[0]
    r = 0 if v is None else v.shape[1]
    hd = [[(-1.0) ** bin(i & j).count("1") / np.sqrt(128) for j in range(128)] for i in range(128)]

    def rot(row):  # row-vector times blockdiag(H)
        out = [0.0] * k
        for blk in range(k // 128):
            for j in range(128):
                out[blk * 128 + j] = sum(row[blk * 128 + i] * hd[i][j] for i in range(128))
        return out

    vv = [[float(v[i, c]) for c in range(r)] for i in range(k)] if r else []
    proj = [[(1.0 if i == j else 0.0) - sum(vv[i][c] * vv[j][c] for c in range(r))
             for j in range(k)] for i in range(k)]

    def side(row):
        u = [sum(row[i] * vv[i][c] for i in range(k)) for c in range(r)]
        d = [sum(row[i] * proj[i][j] for i in range(k)) for j in range(k)]
        d32 = np.array(d, dtype=np.float32)
        q = []
        for blk in range(k // 16):
            q += _bf_quant_block(d32[blk * 16:(blk + 1) * 16])
        return u, q

    wt = [rot([float(w[o, i]) * float(s[i]) for i in range(k)]) for o in range(n)]
    if not shared:
        wside = [side(row) for row in wt]
    else:
        # shared-weight arm: the rotated weight itself is quantised, and the
        # low-rank factor is that decoded weight times V
        wside = []
        for row in wt:
            r32 = np.array(row, dtype=np.float32)
            q = []
            for blk in range(k // 16):
                q += _bf_quant_block(r32[blk * 16:(blk + 1) * 16])
            lw = [sum(q[i] * vv[i][c] for i in range(k)) for c in range(r)]
            wside.append((lw, q))
    y = np.zeros((m, n))
    for a in range(m):
        xt = rot([float(x[a, i]) / float(s[i]) for i in range(k)])
        u, xq = side(xt)
        ub = A.round_bf16(np.array(u)) if r else []
        for o in range(n):
            lw, wq = wside[o]
            acc = sum(xq[i] * wq[i] for i in range(k))
            acc += sum(ub[c] * float(A.round_bf16(lw[c])) for c in range(r))
            y[a, o] = acc + float(b[o])
    return y


@pytest.mark.parametrize("m,r", [(1, 0), (2, 1), (3, 2), (2, 4)])
def test_brute_force_tiny_layers(m, r):
    lay = synth.make_layer("tiny", m, 128, 16, r, seed=100 + 10 * m + r, dtype="f32")
    y = A.forward(lay.x, lay.w, lay.b, lay.s, lay.v)
    yb = _bf_forward(lay.x, lay.w, lay.b, lay.s, lay.v)
    assert np.abs(y - yb).max() <= 1e-9 * np.abs(yb).max()


@pytest.mark.parametrize("m,r", [(1, 1), (2, 3)])
def test_brute_force_tiny_layers_shared_weight(m, r):
    lay = synth.make_layer("tiny", m, 128, 16, r, seed=200 + 10 * m + r, dtype="f32")
    y = A.forward(lay.x, lay.w, lay.b, lay.s, lay.v, form="shared")
    yb = _bf_forward(lay.x, lay.w, lay.b, lay.s, lay.v, shared=True)
    assert np.abs(y - yb).max() <= 1e-9 * np.abs(yb).max()


# ------------------------------------------------------- shared-weight arm


@pytest.mark.parametrize("rank", [0, 32])
def test_shared_weight_quantization_off_identity(layer0, rank):
    # the projector on the activation side alone already makes the two terms sum to x W^T
    v = _orthonormal(layer0.v)[:, :rank] if rank else None
    y = A.forward(layer0.x, layer0.w, layer0.b, layer0.s, v, quantize=False, form="shared")
    ref = layer0.x.astype(np.float64) @ layer0.w.astype(np.float64).T + layer0.b
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 1e-12


def test_shared_weight_codes_are_the_undeflated_weight(layer0):
    # one weight: its codes are those of the rank-0 (no subspace) packer
    sh = A.pack_weight(layer0.w, layer0.s, layer0.v, form="shared")
    r0 = A.pack_weight(layer0.w, layer0.s, None)
    assert np.array_equal(sh["w_codes"], r0["w_codes"])
    assert np.array_equal(sh["w_scales"], r0["w_scales"])
    dfl = A.pack_weight(layer0.w, layer0.s, layer0.v)
    assert not np.array_equal(sh["w_codes"], dfl["w_codes"])


def test_shared_weight_equals_deflated_without_subspace(layer0):
    a = A.forward(layer0.x, layer0.w, layer0.b, layer0.s, None, form="shared")
    b = A.forward(layer0.x, layer0.w, layer0.b, layer0.s, None)
    assert np.array_equal(a, b)


def test_unknown_weight_form_rejected(layer0):
    with pytest.raises(ValueError):
        A.pack_weight(layer0.w, layer0.s, layer0.v, form="other")


# ------------------------------------------------------- residency figures


def _golden_residency():
    vals = {}
    path = os.path.join(os.path.dirname(__file__), "golden", "residency.txt")
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            key, val = line.split("=")
            vals[key.strip()] = float(val)
    return vals


def test_residency_matches_model_card():
    g = _golden_residency()
    pk = A.pack_weight(np.ones((32, 256), np.float32), np.ones(256, np.float32))
    per_weight_code = pk["w_codes"].nbytes / (32 * 256)
    per_weight_scale = pk["w_scales"].nbytes / (32 * 256)
    assert per_weight_code * 8 == g["code_bits_per_weight"]
    assert round(g["weights"] * per_weight_code / 2 ** 20) == g["code_mib"]
    assert round(g["weights"] * per_weight_scale / 2 ** 20, 1) == g["scale_mib"]


# ------------------------------------------------- smoothing search (oracle)

from oracle import smoothing as SM  # noqa: E402


def test_smoothing_grid_reading():
    g = SM.grid()
    assert len(g) == 39 and len(set(g)) == 39
    assert g[0] == (0.0, 0.0) and (0.0, 1.0) not in g
    assert all(b == 0.0 or abs(a + b - 1.0) < 1e-12 for a, b in g)
    assert sorted({a for a, _ in g}) == [i / 20 for i in range(20)]


def test_smoothing_vector_by_hand():
    # hand values: sqrt(4)/sqrt(1) = 2, sqrt(1)/sqrt(16) = 1/4, zero maxima -> 1e-5 each:
    # sqrt(1e-5)/sqrt(1e-5) = 1; alpha = 1, beta = 0: the activation maxima themselves
    s = SM.smoothing_vector([4.0, 1.0, 0.0], [1.0, 16.0, 0.0], 0.5, 0.5)
    assert np.array_equal(s, np.float32([2.0, 0.25, 1.0]))
    s = SM.smoothing_vector([3.0, 0.5, 0.0], [7.0, 2.0, 9.0], 1.0, 0.0)
    assert np.array_equal(s, np.float32([3.0, 0.5, 1e-5]))
    assert SM.smoothing_vector([5.0], [2.0], 0.0, 0.0)[0] == 1.0


def test_smoothing_search_brute_force_tiny():
    # the error table from the independent brute-force layer
    lay = synth.make_layer("tiny", 2, 128, 8, 2, seed=301, dtype="f32")
    cands = [(0.0, 0.0), (0.5, 0.5), (0.9, 0.0)]
    mse, best = SM.search(lay.x, lay.w, lay.b, lay.v, cands)
    x64 = lay.x.astype(np.float64)
    ref = x64 @ lay.w.astype(np.float64).T + lay.b
    want = []
    for a, b in cands:
        xm, wm = np.abs(x64).max(axis=0), np.abs(lay.w.astype(np.float64)).max(axis=0)
        s = ((xm ** a) / (wm ** b)).astype(np.float32)
        want.append(np.mean((_bf_forward(lay.x, lay.w, lay.b, s, lay.v) - ref) ** 2))
    want = np.array(want)
    assert np.allclose(mse, want, rtol=1e-9, atol=0)
    assert best == int(np.argmin(want))
