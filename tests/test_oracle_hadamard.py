"""Pins for the oracle's block Hadamard rotation (CPU only).

Model card "FastWAM UR3 3-task -- 4-bit quantisations", section "What ASP is,
and what the deflated form means": x_tilde = (x / s) H with H a block Hadamard.
Pinned against the closed form H[i, j] = (-1)^popcount(i & j) of the Sylvester
ordering, orthogonality, the 2 x 2 base case and an explicit Kronecker-product
block-diagonal matrix.
"""

import numpy as np
import pytest

from oracle import hadamard as Hd


def test_base_cases():
    assert Hd.sylvester(1).tolist() == [[1.0]]
    assert Hd.sylvester(2).tolist() == [[1.0, 1.0], [1.0, -1.0]]


def test_closed_form_sylvester_order():
    n = 128
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    pop = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    assert np.array_equal(Hd.sylvester(n), (-1.0) ** pop)


def test_orthogonal_symmetric():
    h = Hd.sylvester(128)
    assert np.array_equal(h @ h.T, 128 * np.eye(128))
    assert np.array_equal(h, h.T)
    hn = Hd.normalized(128)
    assert np.abs(hn @ hn.T - np.eye(128)).max() < 1e-15


def test_block_rotation_is_kronecker_block_diagonal():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 384))
    dense = np.kron(np.eye(3), Hd.sylvester(128)) / np.sqrt(128)
    assert np.abs(Hd.block_rotate(x) - x @ dense).max() < 1e-12


def test_rotation_is_an_involution_and_maps_unit_vectors_to_columns():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 256))
    assert np.abs(Hd.block_rotate(Hd.block_rotate(x)) - x).max() < 1e-13
    e = np.zeros((1, 256))
    e[0, 130] = 1.0  # channel 2 of the second block
    got = Hd.block_rotate(e)
    assert np.all(got[0, :128] == 0)
    assert np.array_equal(got[0, 128:] * np.sqrt(128), Hd.sylvester(128)[2])


def test_rejects_bad_sizes():
    with pytest.raises(ValueError):
        Hd.sylvester(12)
    with pytest.raises(ValueError):
        Hd.block_rotate(np.zeros((1, 200)))
