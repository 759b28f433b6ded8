"""Block Hadamard rotation for the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The model card "FastWAM UR3 3-task -- 4-bit quantisations", section "What ASP
is, and what the deflated form means", rotates the smoothed activation by "a
block Hadamard" H: x_tilde = (x / s) H.  The page fixes neither the block size
nor the ordering.  Reading taken here: blocks of 128 consecutive channels, each
the Sylvester-ordered Hadamard matrix scaled by 1/sqrt(128), so H is symmetric
and orthogonal (H = H^T, H H^T = I).
"""

import numpy as np

HADAMARD_BLOCK = 128


def sylvester(n: int) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix of order n (a power of two).

    Built by the doubling rule H_2n = [[H_n, H_n], [H_n, -H_n]] from H_1 = [1].
    """
    if n < 1 or n & (n - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def normalized(n: int = HADAMARD_BLOCK) -> np.ndarray:
    """Orthonormal Sylvester Hadamard matrix, H / sqrt(n)."""
    return sylvester(n) / np.sqrt(n)


def block_rotate(x, block: int = HADAMARD_BLOCK) -> np.ndarray:
    """Right-multiply every row of x by blockdiag(H_block, ..., H_block).

    x: (rows, K) with K a multiple of ``block``.  Returns float64.  Block j acts
    on channels [j*block, (j+1)*block).  Since H is symmetric this is also
    x @ H^T, i.e. the rotation applied to row vectors.
    """
    x = np.asarray(x, dtype=np.float64)
    rows, k = x.shape
    if k % block:
        raise ValueError("K must be a multiple of the Hadamard block")
    h = normalized(block)
    return (x.reshape(rows, k // block, block) @ h).reshape(rows, k)
