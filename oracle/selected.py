"""fp64 oracle for the row/column-selected Muon step with error feedback.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Parity status: pinned
by ``tests/test_oracle_selected.py`` (brute-force subset selection on tiny
inputs, the full-selection reduction to the plain step, the one-row closed
form, exact error-feedback accumulation, permutation equivariance and the
transpose relation).

Source: Dion3 review (blog.secrett2633.cloud), §3 "Method & Key Results":
the update rule uses only part of the rows / columns of the momentum matrix
to shrink the orthogonalisation; §1 "Key Terms & Definitions", Error
Feedback: the error of a reduced-size approximation is carried into later
steps instead of being dropped.  The page gives no formula; the readings
below are the plainest ones both statements support:

  * selection runs along the short side: with m = min(rows, cols), the
    "rows" are those of the oriented m×n matrix (stored rows of a wide or
    square matrix, stored columns of a tall one), so the orthogonalised
    block is k×n with k = ⌈ρ·m⌉ and its Gram matrix is k×k;
  * the score of a row is its squared ℓ2 norm; the k largest are kept and
    equal scores are broken by the lower index;
  * error feedback keeps the unused rows in the buffer at full weight:
        B = M + g,
        O_S = NS_s(B_S / (‖B_S‖_F + eps))          (B_S the selected rows),
        W_S ← round(W_S − lr·√max(1, rows/cols)·O_S), other rows unchanged,
        M_S ← β·B_S,  M_rest ← B_rest.
    With ρ = 1 every row is selected, B_t = β·B_{t−1} + g_t and the update
    is the plain step's (the buffer then stores β·B instead of B).
"""

from __future__ import annotations

import math

import numpy as np

from .ns_oracle import bf16_round, lr_shape_scale, muon_orthogonalize


def selected_count(m: int, fraction: float) -> int:
    """k = ⌈ρ·m⌉ rows kept out of m (at least one when m ≥ 1), with ρ·m
    formed in fp64."""
    if m == 0:
        return 0
    return max(1, min(m, int(math.ceil(float(fraction) * m))))


def select_rows(scores, k: int) -> np.ndarray:
    """Indices of the k largest scores in ascending index order; among
    equal scores the lower index is taken first."""
    s = np.asarray(scores)
    order = sorted(range(len(s)), key=lambda i: (-s[i], i))
    return np.array(sorted(order[:k]), dtype=np.int64)


def row_scores(B) -> np.ndarray:
    """Squared ℓ2 norm of every row of an m×n matrix, in fp64."""
    B = np.asarray(B, dtype=np.float64)
    return np.sum(B * B, axis=1)


def muon_step_selected(W, g, M, beta, lr, coeffs, steps, eps, fraction, scores=None):
    """One selected-row Muon step for one matrix (stored rows × cols).

    W: weights (values of a bf16 tensor), g: fp32 gradient, M: fp32 buffer.
    Returns (W_new as fp64 bf16 values, M_new fp32, S, O_S fp64) where S are
    the selected indices along the short side and O_S the orthogonalised
    selected block in the oriented (k×n) layout.

    ``scores`` replaces the fp64 row scores when the caller fixes the
    selection precision (tests whose scores are well separated do not)."""
    W = np.asarray(W, dtype=np.float64)
    rows, cols = W.shape
    B32 = (np.asarray(M, dtype=np.float64) + np.asarray(g, dtype=np.float64)).astype(np.float32)
    tall = rows > cols
    Bo = B32.T if tall else B32               # oriented m×n view
    m = Bo.shape[0]
    k = selected_count(m, fraction)
    sc = row_scores(Bo) if scores is None else np.asarray(scores)
    S = select_rows(sc, k)
    XS = Bo[S, :].astype(np.float64)
    OS = muon_orthogonalize(XS, coeffs, steps, eps)
    Wo = (W.T if tall else W).copy()
    lrsc = float(lr) * lr_shape_scale(rows, cols)
    Wo[S, :] = bf16_round(Wo[S, :] - lrsc * OS)
    Mo = Bo.copy()
    Mo[S, :] = (float(beta) * Bo[S, :].astype(np.float64)).astype(np.float32)
    W_new = Wo.T if tall else Wo
    M_new = Mo.T if tall else Mo
    return np.ascontiguousarray(W_new), np.ascontiguousarray(M_new), S, OS
