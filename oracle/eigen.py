"""Top-r eigenspace of a symmetric positive semi-definite matrix, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Model card "FastWAM UR3 3-task -- 4-bit quantisations", section "What ASP is,
and what the deflated form means": the protected basis V of a layer spans the
top eigenspace of the action metric G (the expected J^T J of the action's
sensitivity to the layer input).  G itself needs the trained model and its
calibration data; this takes G as given.  The result has a plain definition,
so the oracle is that definition: the eigenvectors of the r largest
eigenvalues (NumPy's symmetric eigensolver as the library step).

Readings: G is symmetric by construction (an expectation of J^T J), so a G
that is not exactly symmetric is rejected rather than silently symmetrised;
eigenvalues are ordered largest first, equal ones by the solver's order.
"""

import numpy as np


def top_eigenspace(g, r: int):
    """(eigenvalues, descending, length r; orthonormal K x r eigenvectors)."""
    g = np.asarray(g, dtype=np.float64)
    if g.ndim != 2 or g.shape[0] != g.shape[1]:
        raise ValueError("G must be square")
    if not np.array_equal(g, g.T):
        raise ValueError("G must be symmetric")
    if not 1 <= r <= g.shape[0]:
        raise ValueError("r outside [1, K]")
    w, q = np.linalg.eigh(g)
    order = np.argsort(w)[::-1][:r]
    return w[order], q[:, order]


def subspace_distance(v1, v2):
    """Spectral norm of the difference of the two orthogonal projectors: the sine
    of the largest principal angle between the column spans."""
    v1 = np.asarray(v1, dtype=np.float64)
    v2 = np.asarray(v2, dtype=np.float64)
    return np.linalg.norm(v1 @ v1.T - v2 @ v2.T, 2)
