"""Pins for the oracle's top-r eigenspace (CPU only).

Model card "FastWAM UR3 3-task -- 4-bit quantisations", section "What ASP is,
and what the deflated form means": V spans the top eigenspace of the layer's
action metric G.  Q-WAM, Figure 3(b): that metric's leading eigenvalues fall
quickly, which the synthetic metric reproduces.

What pins what:
* a metric built from known eigenpairs (a random orthogonal Q and a shuffled,
  known spectrum): the oracle must return the largest eigenvalues, sorted, and
  their eigenvectors up to sign;
* a diagonal metric (eigenvectors are unit vectors), the 2 x 2 closed form and
  a rank-one metric a a^T (closed form: ||a||^2 along a / ||a||);
* eigenpair invariants on a random PSD metric (G V = V diag(lam), V^T V = I,
  Ritz values equal the trace of V^T G V);
* the projector distance against its closed forms (0 for a rotated basis of the
  same span, 1 for orthogonal spans, sin(theta) for a plane rotation);
* argument checks (non-symmetric G, r outside [1, K]).
"""

import math

import numpy as np
import pytest

from oracle import eigen as E
from wam_asp_w4a4_amd import synth


def _orthogonal(rng, n):
    q, rr = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(rr))


def test_known_eigenpairs_shuffled_spectrum():
    rng = np.random.default_rng(3)
    K, r = 48, 7
    q = _orthogonal(rng, K)
    lam = np.linspace(10.0, 0.5, K)           # distinct, gap 0.2
    perm = rng.permutation(K)                  # eigenvalue order unrelated to column order
    g = (q[:, perm] * lam[perm]) @ q[:, perm].T
    g = 0.5 * (g + g.T)
    w, v = E.top_eigenspace(g, r)
    np.testing.assert_allclose(w, lam[:r], rtol=0, atol=1e-12)
    for i in range(r):
        assert abs(abs(v[:, i] @ q[:, i]) - 1.0) < 1e-10


def test_descending_order_not_ascending():
    g = np.diag([1.0, 5.0, 3.0, 2.0])
    w, v = E.top_eigenspace(g, 2)
    assert list(w) == [5.0, 3.0]
    assert np.allclose(np.abs(v), np.eye(4)[:, [1, 2]])


def test_diagonal_metric_gives_unit_vectors():
    rng = np.random.default_rng(4)
    d = rng.permutation(np.arange(1.0, 33.0))
    w, v = E.top_eigenspace(np.diag(d), 5)
    top = np.argsort(-d)[:5]
    np.testing.assert_array_equal(w, d[top])
    np.testing.assert_allclose(np.abs(v), np.eye(32)[:, top], atol=0)


def test_two_by_two_closed_form():
    a, b, d = 2.0, 0.75, -1.0
    w, v = E.top_eigenspace(np.array([[a, b], [b, d]]), 2)
    m, h = 0.5 * (a + d), math.hypot(0.5 * (a - d), b)
    np.testing.assert_allclose(w, [m + h, m - h], rtol=1e-15)
    # top eigenvector of [[a, b], [b, d]] is proportional to (b, lam1 - a)
    t = np.array([b, m + h - a])
    t /= np.linalg.norm(t)
    assert abs(abs(v[:, 0] @ t) - 1.0) < 1e-14


def test_rank_one_metric():
    rng = np.random.default_rng(5)
    a = rng.standard_normal(20)
    w, v = E.top_eigenspace(np.outer(a, a), 3)
    assert abs(w[0] - a @ a) < 1e-12
    np.testing.assert_allclose(w[1:], 0.0, atol=1e-12)
    assert abs(abs(v[:, 0] @ a) / np.linalg.norm(a) - 1.0) < 1e-12


def test_eigenpair_invariants_random_psd():
    rng = np.random.default_rng(6)
    j = rng.standard_normal((200, 64))
    g = j.T @ j
    g = 0.5 * (g + g.T)
    w, v = E.top_eigenspace(g, 12)
    np.testing.assert_allclose(g @ v, v * w, atol=1e-9 * w[0])
    np.testing.assert_allclose(v.T @ v, np.eye(12), atol=1e-13)
    assert abs(np.trace(v.T @ g @ v) - w.sum()) < 1e-10 * w[0]
    assert np.all(np.diff(w) <= 0)
    # Ky Fan: the top-r eigenvalue sum bounds the trace over any r-dim subspace
    u = np.linalg.qr(rng.standard_normal((64, 12)))[0]
    assert np.trace(u.T @ g @ u) <= w.sum() + 1e-9


def test_synthetic_metric_spectrum_is_its_eigenvalues():
    rng = np.random.default_rng(7)
    g, lam, q = synth.draw_metric(rng, 64, decay=4.0)
    assert g.dtype == np.float32 and np.array_equal(g, g.T)
    w, v = E.top_eigenspace(g, 8)
    # float32 rounding of G moves eigenvalues by at most ||dG||_2 <= ||dG||_F
    bound = np.linalg.norm(g.astype(np.float64) - (q * lam) @ q.T)
    np.testing.assert_allclose(w, lam[:8], rtol=0, atol=bound + 1e-15)


def test_projector_distance_closed_forms():
    rng = np.random.default_rng(8)
    v = np.linalg.qr(rng.standard_normal((30, 4)))[0]
    rot = _orthogonal(rng, 4)
    assert E.subspace_distance(v, v @ rot) < 1e-14
    e = np.eye(30)
    assert abs(E.subspace_distance(e[:, :2], e[:, 2:4]) - 1.0) < 1e-15
    th = 0.3
    v2 = (math.cos(th) * e[:, 0] + math.sin(th) * e[:, 1])[:, None]
    assert abs(E.subspace_distance(e[:, :1], v2) - math.sin(th)) < 1e-15


def test_argument_checks():
    g = np.array([[1.0, 2.0], [2.0 + 1e-12, 1.0]])
    with pytest.raises(ValueError):
        E.top_eigenspace(g, 1)
    with pytest.raises(ValueError):
        E.top_eigenspace(np.eye(3), 0)
    with pytest.raises(ValueError):
        E.top_eigenspace(np.eye(3), 4)


def test_reflected_metric_has_its_stated_eigenpairs():
    """The large-K test metric (Householder reflections applied to a known
    spectrum): the returned columns are orthonormal, exact symmetric
    eigenvectors of the float32 metric up to its rounding, and the oracle's
    eigensolver finds the same leading eigenvalues at a size it can afford."""
    rng = np.random.default_rng(5)
    g, lam, q = synth.draw_metric_reflected(rng, 384, 12)
    assert np.array_equal(g, g.T)
    assert np.abs(q.T @ q - np.eye(12)).max() <= 1e-14
    g64 = g.astype(np.float64)
    fro = np.linalg.norm(g64)
    assert np.abs(g64 @ q - q * lam[:12]).max() <= 2.0 ** -24 * fro * 4
    w, v = E.top_eigenspace(g, 12)
    assert np.abs(w - lam[:12]).max() <= 2.0 ** -24 * fro * 4
    assert E.subspace_distance(v, q) <= 1e-6
