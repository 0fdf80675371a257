"""Exact rational-arithmetic versions of the two NS recursions, on tiny
integer matrices (lists of lists of ``fractions.Fraction``).

TEST INFRASTRUCTURE ONLY.  Used to show, with no rounding at all, that the
Gram-space recursion of DMuon's technical summary (gist.science, Korean,
§2.2) returns exactly what the standard m×n-space iteration returns, and that
every Gram-space iterate is symmetric.  No normalisation here (a square root
is not rational); the algebra does not need it.
"""

from __future__ import annotations

from fractions import Fraction


def mat(rows):
    return [[Fraction(v) for v in r] for r in rows]


def transpose(X):
    return [list(col) for col in zip(*X)]


def matmul(X, Y):
    n_in = len(Y)
    assert all(len(r) == n_in for r in X)
    cols = len(Y[0])
    return [[sum((X[i][k] * Y[k][j] for k in range(n_in)), Fraction(0))
             for j in range(cols)] for i in range(len(X))]


def add(X, Y):
    return [[x + y for x, y in zip(rx, ry)] for rx, ry in zip(X, Y)]


def scale(s, X):
    return [[s * x for x in r] for r in X]


def eye(m):
    return [[Fraction(int(i == j)) for j in range(m)] for i in range(m)]


def standard_ns(X, coeffs, steps):
    """X ← a·X + (b·A + c·A²)·X, A = X·Xᵀ, exactly."""
    a, b, c = coeffs
    for _ in range(steps):
        A = matmul(X, transpose(X))
        B = add(scale(b, A), scale(c, matmul(A, A)))
        X = add(scale(a, X), matmul(B, X))
    return X


def gram_ns(X0, coeffs, steps, record=None):
    """A₀ = X₀·X₀ᵀ, Q₀ = I; P = a·I + b·A + c·A²; Q ← P·Q; A ← P·A·P;
    result Q·X₀, exactly.  If ``record`` is a list, every Gram-space matrix
    formed (A, A², P, Q, P·A, P·A·P) is appended to it."""
    a, b, c = coeffs
    m = len(X0)
    I = eye(m)
    A = matmul(X0, transpose(X0))
    Q = I
    if record is not None:
        record.append(A)
    for _ in range(steps):
        A2 = matmul(A, A)
        P = add(add(scale(a, I), scale(b, A)), scale(c, A2))
        Q = matmul(P, Q)
        PA = matmul(P, A)
        A = matmul(P, PA)
        if record is not None:
            record.extend([A2, P, Q, PA, A])
    return matmul(Q, X0)
