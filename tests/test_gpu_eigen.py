"""Device top-r eigenspace against the oracle (numpy's symmetric eigensolver on
the same float32 metric), through the C ABI.

Gates, from the arithmetic (float64 throughout on the device, float32 outputs):
* eigenvalues: |theta_i - lam_i| <= 2^-23 |lam_i| + 1e-9 lam_1 (the float32
  rounding of the output plus float64 accumulation over K terms);
* eigenvectors: for each returned column, the sine of its angle to the
  oracle's eigenvector (or, inside a cluster of equal eigenvalues, to the
  cluster's span) <= 1e-5, and the projector distance of the whole subspace
  <= 1e-5: float32 rounding gives ~1e-7, the iteration counts below leave a
  convergence error below 1e-8 for the spectra used;
* every output: orthonormal columns to 1e-6, the largest-magnitude entry of
  each column positive, residual norms <= 1e-6 lam_1, results bitwise equal
  run to run.
"""

import numpy as np
import pytest
import torch

from oracle import eigen as E
from wam_asp_w4a4_amd import binding as B
from wam_asp_w4a4_amd import synth
from wam_asp_w4a4_amd.layer import top_eigenspace

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(g, v0, r, iters):
    gd = torch.from_numpy(np.ascontiguousarray(g, np.float32)).to(DEV)
    vd = torch.from_numpy(np.ascontiguousarray(v0, np.float32)).to(DEV)
    v, ev, res = top_eigenspace(gd, vd, r, iters)
    torch.cuda.synchronize()
    return v.cpu().numpy().astype(np.float64), ev.cpu().numpy().astype(np.float64), \
        res.cpu().numpy().astype(np.float64)


def sine(v, q):
    """Sine of the angle between column v and the span of q's columns."""
    v = v / np.linalg.norm(v)
    return float(np.linalg.norm(v - q @ (q.T @ v)))


def check_common(g, v, ev, res, lam1):
    K, r = v.shape
    assert np.abs(v.T @ v - np.eye(r)).max() <= 1e-6
    idx = np.argmax(np.abs(v), axis=0)
    assert np.all(v[idx, np.arange(r)] > 0)
    assert np.all(np.diff(ev) <= 0)
    assert res.max() <= 1e-6 * lam1 + 1e-30
    # residuals recomputed on the host from the float32 outputs
    host_res = np.linalg.norm(g.astype(np.float64) @ v - v * ev, axis=0)
    assert host_res.max() <= 1e-6 * lam1 + 1e-30


def check_against_oracle(g, v, ev, res, r, clusters=None):
    w, q = E.top_eigenspace(g, r)
    lam1 = abs(w[0])
    check_common(g, v, ev, res, lam1)
    assert np.all(np.abs(ev - w) <= 2.0 ** -23 * np.abs(w) + 1e-9 * lam1), (ev[:4], w[:4])
    clusters = clusters or [[i] for i in range(r)]
    for c in clusters:
        for i in c:
            assert sine(v[:, i], q[:, c]) <= 1e-5, (i, sine(v[:, i], q[:, c]))
    assert E.subspace_distance(v, q) <= 1e-5


CASES = [
    # K, p, r, iters, decay
    (512, 64, 32, 8, 8.0),
    (384, 48, 5, 12, 4.0),
    (1024, 32, 16, 10, 4.0),
    (128, 16, 4, 30, 2.0),
]


@pytest.mark.parametrize("K,p,r,iters,decay", CASES)
def test_eigenspace_matches_oracle(K, p, r, iters, decay):
    print(f"eigenspace K={K} p={p} r={r} iters={iters} decay={decay}", flush=True)
    rng = np.random.default_rng(K + p + r)
    g, lam, _ = synth.draw_metric(rng, K, decay=decay)
    v0 = synth.draw_start(rng, K, p)
    v, ev, res = run(g, v0, r, iters)
    check_against_oracle(g, v, ev, res, r)


def test_block_equal_to_rank_with_gap():
    """r = p (no oversampling): converges when the spectrum has a gap at r."""
    print("eigenspace r = p = 16, gapped", flush=True)
    rng = np.random.default_rng(11)
    K = 256
    q, _ = np.linalg.qr(rng.standard_normal((K, K)))
    lam = np.concatenate([np.linspace(2.0, 1.0, 16), 1e-3 * np.exp(-np.arange(K - 16) / 10)])
    g = (q * lam) @ q.T
    g = (0.5 * (g + g.T)).astype(np.float32)
    v, ev, res = run(g, synth.draw_start(rng, K, 16), 16, 8)
    check_against_oracle(g, v, ev, res, 16)


def test_repeated_eigenvalues():
    """A cluster of three equal eigenvalues: only the cluster's span is unique."""
    print("eigenspace repeated eigenvalues", flush=True)
    rng = np.random.default_rng(12)
    K = 256
    q, _ = np.linalg.qr(rng.standard_normal((K, K)))
    lam = np.concatenate([[9.0, 5.0, 5.0, 5.0, 3.0], 0.5 * np.exp(-np.arange(K - 5) / 4)])
    g = (q * lam) @ q.T
    g = (0.5 * (g + g.T)).astype(np.float32)
    v, ev, res = run(g, synth.draw_start(rng, K, 32), 5, 10)
    # the float32 rounding of G splits the cluster by ~1e-6, so compare spans
    check_against_oracle(g, v, ev, res, 5, clusters=[[0], [1, 2, 3], [4]])


def test_zero_metric():
    print("eigenspace G = 0", flush=True)
    rng = np.random.default_rng(13)
    K, p, r = 256, 16, 6
    g = np.zeros((K, K), np.float32)
    v, ev, res = run(g, synth.draw_start(rng, K, p), r, 3)
    assert np.all(ev == 0.0) and np.all(res == 0.0)
    assert np.abs(v.T @ v - np.eye(r)).max() <= 1e-6


def test_rank_deficient_metric():
    """rank(G) = 3 < r: the top three pairs are unique; the rest have eigenvalues
    ~0 (float32 rounding of G) and need only be orthonormal Ritz pairs inside
    that cluster."""
    print("eigenspace rank 3", flush=True)
    rng = np.random.default_rng(14)
    K = 128
    a = rng.standard_normal((K, 3))
    g = a @ a.T
    g = (0.5 * (g + g.T)).astype(np.float32)
    v, ev, res = run(g, synth.draw_start(rng, K, 16), 8, 6)
    w, q = E.top_eigenspace(g, 8)
    check_common(g, v, ev, res, w[0])
    tol = 2.0 ** -23 * np.abs(w) + 1e-9 * w[0]
    assert np.all(np.abs(ev[:3] - w[:3]) <= tol[:3])
    assert E.subspace_distance(v[:, :3], q[:, :3]) <= 1e-5
    # beyond the rank: G's float32 rounding leaves ~K - 3 eigenvalues of order
    # 1e-6 lam_1 whose eigenvectors are not determined; the device's Ritz values
    # must only lie inside that cluster
    lo = np.linalg.eigvalsh(g.astype(np.float64))[0]
    assert np.all(ev[3:] <= w[3] + tol[3]) and np.all(ev[3:] >= lo - tol[3])


def test_no_iterations_gives_ritz_pairs_of_the_start():
    """iters = 0: the Rayleigh-Ritz pairs of span(V0) -- V lies in span(V0) and
    V^T G V is diagonal with the returned eigenvalues (properties at any size)."""
    print("eigenspace iters = 0", flush=True)
    rng = np.random.default_rng(15)
    K, p, r = 512, 32, 32
    g, _, _ = synth.draw_metric(rng, K)
    v0 = synth.draw_start(rng, K, p)
    v, ev, res = run(g, v0, r, 0)
    q0, _ = np.linalg.qr(v0.astype(np.float64))
    assert np.linalg.norm(v - q0 @ (q0.T @ v)) <= 1e-5
    t = v.T @ g.astype(np.float64) @ v
    lam1 = np.linalg.eigvalsh(g.astype(np.float64)).max()
    assert np.abs(t - np.diag(ev)).max() <= 1e-6 * lam1
    # oracle Rayleigh-Ritz of the same span: eigenvalues of Q0^T G Q0
    w = np.sort(np.linalg.eigvalsh(q0.T @ g.astype(np.float64) @ q0))[::-1][:r]
    assert np.all(np.abs(ev - w) <= 2.0 ** -23 * np.abs(w) + 1e-9 * lam1)


def test_bitwise_reproducible():
    print("eigenspace reproducibility", flush=True)
    rng = np.random.default_rng(16)
    g, _, _ = synth.draw_metric(rng, 512)
    v0 = synth.draw_start(rng, 512, 64)
    a = run(g, v0, 32, 5)
    b = run(g, v0, 32, 5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_non_finite_metric_reports_nan():
    print("eigenspace non-finite G", flush=True)
    rng = np.random.default_rng(17)
    g, _, _ = synth.draw_metric(rng, 128)
    g[5, 7] = g[7, 5] = np.nan
    _, ev, _ = run(g, synth.draw_start(rng, 128, 16), 4, 2)
    assert np.all(np.isnan(ev))


def test_full_size_action_metric():
    """K = 4096 (the action expert's widest input), p = 64, r = 32, 8 iterations:
    the configuration the benchmark times.  The oracle's eigh at this size is
    run once; its eigenpairs gate the device result as above."""
    print("eigenspace K=4096 p=64 r=32", flush=True)
    rng = np.random.default_rng(18)
    g, lam, _ = synth.draw_metric(rng, 4096)
    v0 = synth.draw_start(rng, 4096, 64)
    v, ev, res = run(g, v0, 32, 8)
    check_against_oracle(g, v, ev, res, 32)


def test_large_metric_known_spectrum():
    """K = 16384, p = 64, r = 32: a metric built from four Householder
    reflections, so its spectrum and leading eigenvectors are known without an
    eigh at this size.  Against the exact float64 eigenpairs the float32
    rounding of G (||dG||_2 <= ||dG||_F <= 2^-24 ||G||_F) moves each
    eigenvalue by at most that much (Weyl) and the r-dimensional subspace by
    at most that over the gap lam_r - lam_{r+1} (Davis-Kahan); the gates add
    those bounds to the ones above.  Orthonormality, signs and residuals as
    for every case."""
    print("eigenspace K=16384 p=64 r=32 (reflected metric)", flush=True)
    K, p, r = 16384, 64, 32
    rng = np.random.default_rng(23)
    g, lam, q = synth.draw_metric_reflected(rng, K, r)
    v0 = synth.draw_start(rng, K, p)
    v, ev, res = run(g, v0, r, 8)
    check_common(g, v, ev, res, lam[0])
    dg = 2.0 ** -24 * float(np.linalg.norm(g.astype(np.float64)))
    assert np.all(np.abs(ev - lam[:r]) <= 2.0 ** -23 * lam[:r] + dg + 1e-9 * lam[0]), ev[:4]
    # the largest sine of the principal angles, as the 2-norm of the part of v
    # outside span(q) (linear in the error; sqrt(1 - s_min^2) would turn the
    # float32 rounding of v's orthonormality, about 1e-8, into 1e-4)
    dist = float(np.linalg.norm(v - q @ (q.T @ v), 2))
    bound = dg / (lam[r - 1] - lam[r]) + 1e-6
    print(f"  subspace distance {dist:.2e} (bound {bound:.2e}), "
          f"max eigenvalue error {np.abs(ev - lam[:r]).max():.2e} (dG {dg:.2e})")
    assert dist <= bound


@pytest.mark.parametrize("K,p", [(4096, 64), (1024, 48), (384, 16)])
def test_metric_product_partials(K, p):
    """The MFMA product alone: the slices' partial sums add up to G V (float64
    reference product of the same float32 G and float64 V); each slice is a
    K/S-term float64 dot product, so the error is ~1e-15 of |G| |V|."""
    print(f"metric product K={K} p={p}", flush=True)
    rng = np.random.default_rng(K + p)
    g = rng.standard_normal((K, K)).astype(np.float32)
    v = rng.standard_normal((K, p))
    S = B.asp_top_eigenspace_slices(K, p)
    yp = torch.empty((S, K, p), dtype=torch.float64, device=DEV)
    B.asp_metric_product_partials(torch.from_numpy(g).to(DEV), K,
                                  torch.from_numpy(v).to(DEV), p, yp)
    torch.cuda.synchronize()
    parts = yp.cpu().numpy()
    g64 = g.astype(np.float64)
    scale = np.abs(g64) @ np.abs(v)
    for s in range(S):
        sl = slice(s * K // S, (s + 1) * K // S)
        want = g64[:, sl] @ v[sl]
        assert np.all(np.abs(parts[s] - want) <= 1e-13 * scale), s
