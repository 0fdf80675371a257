"""fp64 oracle for the Muon step with Newton–Schulz orthogonalisation.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Parity status: every
function here is pinned by ``tests/test_oracle.py`` against closed forms,
exact rational arithmetic, LAPACK's SVD and invariants of the iteration.

Sources (the pages):
  * DMuon technical summary (gist.science, Korean), §1 "Problem definition":
    Muon applies a Newton–Schulz (NS) iteration to the momentum-accumulated
    gradient of each weight matrix; the iteration needs the product X·Xᵀ.
  * same page, §2.2 "Efficient Gram Newton–Schulz iteration": the recursion
    can run on the m×m Gram matrix G = X·Xᵀ instead of the m×n matrix when
    m < n; G is symmetric.
  * DeMuon technical summary (gist.science, Korean), Method §1: the local
    momentum is an exponentially weighted moving average of stochastic
    gradients, and the update applies the matrix sign msgn(·).
  * DMuon page (gist.science, Japanese), technical summary §1: NS drives the
    update's singular values toward a uniform spectrum.

Readings where the pages are silent (the same readings the HIP library
implements, stated here so the oracle can be checked on its own):
  * polynomial form: X ← a·X + (b·A + c·A²)·X with A = X·Xᵀ, so each singular
    value maps σ ↦ aσ + bσ³ + cσ⁵;
  * normalisation: X₀ = M / (‖M‖_F + eps);
  * orientation: a matrix with rows > cols is transposed before the
    iteration and transposed back after it;
  * momentum: M ← β·M + g (accumulating form; the EMA form differs by the
    factor (1−β), which the normalisation removes);
  * weight update: W ← round_bf16(W − lr·√max(1, rows/cols)·O), no weight
    decay, computed in fp64 and rounded once.
"""

from __future__ import annotations

import math

import numpy as np

# Quintic coefficients (5 steps) and the convergent cubic (a, b, c); the
# pages give none, these are the workload's stated coefficient sets.
QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), once.

    bfloat16 keeps 8 significant bits and the float32 exponent range.  The
    value is split as f·2**e with 0.5 ≤ |f| < 1, f·2**8 is rounded half to
    even and scaled back.  Values beyond the bf16 range become ±inf; the
    bf16 subnormal range is not modelled (not reached by the workloads).
    """
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    r = np.ldexp(np.rint(f * 256.0), e - 8)
    max_bf16 = float(np.ldexp(255.0, 127 - 7))  # (2 - 2**-7) * 2**127
    r = np.where(np.abs(r) > max_bf16, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def frobenius_normalize(x, eps: float) -> np.ndarray:
    """X / (‖X‖_F + eps) in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / (math.sqrt(float(np.sum(x * x))) + eps)


def orient(x) -> tuple[np.ndarray, bool]:
    """Return (X, transposed): X is m×n with m ≤ n (Gram space is m×m)."""
    x = np.asarray(x)
    if x.shape[0] > x.shape[1]:
        return x.T, True
    return x, False


def newton_schulz(X, coeffs, steps: int) -> np.ndarray:
    """Standard m×n-space Newton–Schulz: s times X ← a·X + (b·A + c·A²)·X,
    A = X·Xᵀ.  fp64, numpy matmuls, no reordering."""
    a, b, c = (float(v) for v in coeffs)
    X = np.asarray(X, dtype=np.float64)
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X


def muon_orthogonalize(x, coeffs, steps: int, eps: float) -> np.ndarray:
    """What one matrix of a batched NS call produces: normalise, orient,
    iterate, orient back.  Same shape as ``x``."""
    X0 = frobenius_normalize(x, eps)
    X, transposed = orient(X0)
    O = newton_schulz(X, coeffs, steps)
    return O.T if transposed else O


def polar_svd(X) -> np.ndarray:
    """msgn(X) = U·Vᵀ from LAPACK's compact SVD (DeMuon Method §1: the update
    applies the matrix sign function)."""
    U, _, Vt = np.linalg.svd(np.asarray(X, dtype=np.float64), full_matrices=False)
    return U @ Vt


def scalar_map(sigma, coeffs, steps: int):
    """φ^{∘steps}(σ) with φ(σ) = aσ + bσ³ + cσ⁵ — the action of the
    iteration on one singular value (plain Python floats)."""
    a, b, c = (float(v) for v in coeffs)
    s = float(sigma)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def gram_newton_schulz(X, coeffs, steps: int) -> np.ndarray:
    """The Gram-space recursion in fp64 (DMuon §2.2): with G = X₀·X₀ᵀ,
    A₀ = G, Q₀ = I and P_k = a·I + b·A_k + c·A_k²,
        Q_{k+1} = P_k·Q_k,   A_{k+1} = P_k·A_k·P_k,   O = Q_s·X₀.
    Used only by the algebra checks; the reference result is
    ``newton_schulz``."""
    a, b, c = (float(v) for v in coeffs)
    X0 = np.asarray(X, dtype=np.float64)
    m = X0.shape[0]
    I = np.eye(m)
    A = X0 @ X0.T
    Q = I.copy()
    for _ in range(steps):
        P = a * I + b * A + c * (A @ A)
        Q = P @ Q
        A = P @ A @ P
    return Q @ X0


def momentum_update(M, g, beta: float) -> np.ndarray:
    """M ← β·M + g evaluated in fp64 and rounded once to fp32."""
    M = np.asarray(M, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    return (float(beta) * M + g).astype(np.float32)


def lr_shape_scale(rows: int, cols: int) -> float:
    """√max(1, rows/cols) on the stored (rows × cols) shape."""
    return math.sqrt(max(1.0, rows / cols))


def muon_step(W, g, M, beta, lr, coeffs, steps, eps, nesterov=False, weight_decay=0.0):
    """One Muon step for one matrix.

    W: stored weights (values of a bf16 tensor, any float dtype),
    g: gradient values (fp32, or bf16 values), M: fp32 momentum, all
    rows × cols.  Returns (W_new_bf16_values_as_fp64, M_new_fp32, O_fp64).

    The two options are not part of the pages' method (which is the plain
    step: nesterov False, weight_decay 0); they are the usual Muon-optimiser
    variants, written out here from their definitions:
      nesterov:     the matrix orthogonalised is u = g + β·M' instead of the
                    updated momentum M' (M' is still the returned state);
      weight_decay: decoupled, W' = round((1 − lr·wd)·W − lr·sc·O).
    """
    M_new = momentum_update(M, g, beta)
    U = M_new.astype(np.float64)
    if nesterov:
        U = np.asarray(g, dtype=np.float64) + float(beta) * U
    O = muon_orthogonalize(U, coeffs, steps, eps)
    rows, cols = np.asarray(W).shape
    W64 = np.asarray(W, dtype=np.float64)
    decay = 1.0 - float(lr) * float(weight_decay)
    W_new = bf16_round(decay * W64 - float(lr) * lr_shape_scale(rows, cols) * O)
    return W_new, M_new, O


def gram_flops(rows: int, cols: int, steps: int) -> int:
    """Algorithmic flops of the Gram formulation for one matrix:
    SYRK m(m+1)n + (4s−3)·m²(m+1) symmetric products + 2m²n final product,
    m = min(rows, cols), n = max(rows, cols).  Symmetric products count the
    upper triangle only."""
    m, n = min(rows, cols), max(rows, cols)
    if m == 0 or n == 0:
        return 0
    if steps == 0:
        return 0
    sym = 4 * steps - 3
    return m * (m + 1) * n + sym * m * m * (m + 1) + 2 * m * m * n
