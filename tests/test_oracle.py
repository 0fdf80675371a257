"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: closed forms of the
iteration on a constructed spectrum, exact rational arithmetic, LAPACK's SVD,
invariants of the map, and torch's own bf16 conversion.  The pages print no
worked numeric example, so nothing here is a value taken from them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import rational as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _orth(n, rng):
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))


def _spectral(m, n, sigma, rng):
    U = _orth(m, rng)
    V = _orth(n, rng)[:, :m]
    return U, V, (U * sigma) @ V.T


# -- closed form on a constructed spectrum ----------------------------------

@pytest.mark.parametrize("m,n", [(8, 8), (6, 20), (32, 96)])
@pytest.mark.parametrize("coeffs,steps", [(oracle.QUINTIC, 5), (oracle.CUBIC, 7), ((2.0, -1.5, 0.5), 3)])
def test_standard_ns_acts_on_singular_values(m, n, coeffs, steps):
    """X = U·diag(σ)·Vᵀ ⇒ NS_s(X) = U·diag(φ^s(σ))·Vᵀ with φ(σ)=aσ+bσ³+cσ⁵."""
    rng = np.random.default_rng(m * 1000 + n)
    sigma = np.linspace(0.05, 1.0, m)
    U, V, X = _spectral(m, n, sigma, rng)
    want = (U * np.array([oracle.scalar_map(s, coeffs, steps) for s in sigma])) @ V.T
    got = oracle.newton_schulz(X, coeffs, steps)
    assert np.linalg.norm(got - want) <= 1e-13 * np.linalg.norm(want)


def test_muon_orthogonalize_normalises_by_frobenius_and_orients():
    """Frobenius normalisation divides every σ by √Σσ²; a tall input is the
    transpose of the wide case."""
    rng = np.random.default_rng(7)
    m, n = 5, 12
    sigma = np.array([2.0, 1.5, 1.0, 0.5, 0.25])
    U, V, X = _spectral(m, n, sigma, rng)
    fro = math.sqrt(float(np.sum(sigma ** 2)))
    want = (U * np.array([oracle.scalar_map(s / fro, oracle.QUINTIC, 5) for s in sigma])) @ V.T
    got = oracle.muon_orthogonalize(X, oracle.QUINTIC, 5, eps=0.0)
    assert np.linalg.norm(got - want) <= 1e-13 * np.linalg.norm(want)
    got_t = oracle.muon_orthogonalize(X.T, oracle.QUINTIC, 5, eps=0.0)
    assert got_t.shape == (n, m)
    assert np.linalg.norm(got_t - want.T) <= 1e-13 * np.linalg.norm(want)


def test_scalar_golden_values():
    with open(os.path.join(GOLDEN, "scalar_map.json")) as f:
        gold = json.load(f)
    a, b, c = oracle.QUINTIC
    # φ(1) = a + b + c by hand.
    assert gold["quintic_phi1_of_1"] == pytest.approx(a + b + c, abs=1e-15)
    assert gold["quintic_phi1_of_1"] == pytest.approx(0.701, abs=1e-12)
    # φ^5(1) by iterating the cubic-in-σ² polynomial written out here.
    s = 1.0
    for _ in range(5):
        s2 = s * s
        s = s * (a + s2 * (b + c * s2))
    assert gold["quintic_phi5_of_1"] == pytest.approx(s, rel=1e-14)
    assert oracle.scalar_map(1.0, oracle.QUINTIC, 5) == pytest.approx(gold["quintic_phi5_of_1"], rel=1e-15)
    # The cubic map has the fixed point 1 and pulls small σ there.
    assert gold["cubic_phi30_of_0.05"] == pytest.approx(1.0, abs=1e-12)


def test_row_vector_closed_form():
    """m = 1: after normalisation σ = 1, so O = φ^5(1)·x/‖x‖."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((1, 37))
    got = oracle.muon_orthogonalize(x, oracle.QUINTIC, 5, eps=0.0)
    want = oracle.scalar_map(1.0, oracle.QUINTIC, 5) * x / np.linalg.norm(x)
    assert np.allclose(got, want, rtol=1e-14, atol=1e-16)
    # and as a column (tall, transposed internally)
    got_c = oracle.muon_orthogonalize(x.T, oracle.QUINTIC, 5, eps=0.0)
    assert np.allclose(got_c, want.T, rtol=1e-14, atol=1e-16)


# -- cubic iteration vs SVD polar factor -------------------------------------

def test_cubic_30_steps_matches_svd_polar():
    """(1.5, −0.5, 0) for 30 steps on the normalised 256×1024 Gaussian reaches
    msgn(X) = U·Vᵀ (DeMuon Method §1)."""
    rng = np.random.default_rng(1001)
    X = rng.standard_normal((256, 1024))
    got = oracle.muon_orthogonalize(X, oracle.CUBIC, 30, eps=0.0)
    want = oracle.polar_svd(X)
    assert np.linalg.norm(got - want) <= 1e-12 * np.linalg.norm(want)


def test_polar_svd_properties():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((6, 15))
    P = oracle.polar_svd(X)
    assert np.allclose(P @ P.T, np.eye(6), atol=1e-13)
    # X = P·(XᵀX)^{1/2} restricted to the row space: P·Xᵀ is symmetric PSD
    S = P @ X.T
    assert np.allclose(S, S.T, atol=1e-12)
    assert np.all(np.linalg.eigvalsh((S + S.T) / 2) > 0)


def test_quintic_does_not_reach_polar_factor():
    """The quintic set is not convergent: φ(1)=0.701, so five steps leave the
    output measurably away from U·Vᵀ (parity for it is against standard NS)."""
    rng = np.random.default_rng(1001)
    X = rng.standard_normal((256, 1024))
    got = oracle.muon_orthogonalize(X, oracle.QUINTIC, 5, eps=0.0)
    err = np.linalg.norm(got - oracle.polar_svd(X)) / np.linalg.norm(oracle.polar_svd(X))
    assert 0.05 < err < 0.4


# -- Gram recursion ≡ standard recursion --------------------------------------

@pytest.mark.parametrize("X,steps", [
    ([[1, 2, 0], [-1, 1, 3]], 2),
    ([[1, 0, 2, -1, 1], [0, 1, 1, 1, -2], [2, -1, 0, 1, 1]], 2),
    ([[1, -1, 0], [2, 1, 1]], 3),
])
@pytest.mark.parametrize("coeffs", [
    (Fraction(6889, 2000), Fraction(-191, 40), Fraction(4063, 2000)),  # 3.4445, −4.775, 2.0315
    (Fraction(3, 2), Fraction(-1, 2), Fraction(0)),
])
def test_gram_equals_standard_exactly(X, steps, coeffs):
    X = R.mat(X)
    assert R.gram_ns(X, coeffs, steps) == R.standard_ns(X, coeffs, steps)


def test_rational_coefficients_are_the_quintic():
    assert float(Fraction(6889, 2000)) == oracle.QUINTIC[0]
    assert float(Fraction(-191, 40)) == oracle.QUINTIC[1]
    assert float(Fraction(4063, 2000)) == oracle.QUINTIC[2]


def test_every_gram_iterate_is_exactly_symmetric():
    X = R.mat([[1, 0, 2, -1, 1], [0, 1, 1, 1, -2], [2, -1, 0, 1, 1]])
    rec = []
    R.gram_ns(X, (Fraction(6889, 2000), Fraction(-191, 40), Fraction(4063, 2000)), 3, record=rec)
    assert len(rec) == 1 + 5 * 3
    for Y in rec:
        assert Y == R.transpose(Y)
    # products of two commuting iterates are symmetric too (B·Q, B·A, B·PA)
    A, A2, P, Q = rec[0], rec[1], rec[2], rec[3]
    for Y, Z in [(P, Q), (P, A), (A2, A), (P, R.matmul(P, A))]:
        YZ = R.matmul(Y, Z)
        assert YZ == R.transpose(YZ)


def test_gram_fp64_matches_standard_fp64():
    rng = np.random.default_rng(64)
    X = oracle.frobenius_normalize(rng.standard_normal((64, 256)), 0.0)
    a = oracle.gram_newton_schulz(X, oracle.QUINTIC, 5)
    b = oracle.newton_schulz(X, oracle.QUINTIC, 5)
    assert np.linalg.norm(a - b) <= 1e-12 * np.linalg.norm(b)


def test_fp64_gram_iterates_symmetric():
    rng = np.random.default_rng(5)
    X = oracle.frobenius_normalize(rng.standard_normal((48, 160)), 0.0)
    a, b, c = oracle.QUINTIC
    A = X @ X.T
    I = np.eye(48)
    Q = I
    for _ in range(5):
        A2 = A @ A
        B = b * A + c * A2
        for Y in (A2, B @ Q, B @ A):
            assert np.linalg.norm(Y - Y.T) <= 1e-14 * np.linalg.norm(Y)
        Q = a * Q + B @ Q
        PA = a * A + B @ A
        A = a * PA + B @ PA


# -- invariants ---------------------------------------------------------------

def test_orthonormal_rows_fixed_point_of_cubic():
    rng = np.random.default_rng(9)
    Q, _ = np.linalg.qr(rng.standard_normal((40, 12)))
    X = Q.T  # 12×40 with orthonormal rows
    assert np.allclose(oracle.newton_schulz(X, oracle.CUBIC, 3), X, atol=1e-14)
    got = oracle.muon_orthogonalize(X, oracle.CUBIC, 30, eps=0.0)
    assert np.linalg.norm(got - X) <= 1e-12 * np.linalg.norm(X)


def test_orthogonal_equivariance():
    rng = np.random.default_rng(21)
    X = oracle.frobenius_normalize(rng.standard_normal((10, 30)), 0.0)
    U = _orth(10, rng)
    V = _orth(30, rng)
    lhs = oracle.newton_schulz(U @ X @ V, oracle.QUINTIC, 5)
    rhs = U @ oracle.newton_schulz(X, oracle.QUINTIC, 5) @ V
    assert np.linalg.norm(lhs - rhs) <= 1e-12 * np.linalg.norm(rhs)


def test_odd_scale_transpose_zero_rank():
    rng = np.random.default_rng(31)
    X = rng.standard_normal((12, 40))
    f = lambda Y: oracle.muon_orthogonalize(Y, oracle.QUINTIC, 5, eps=0.0)
    base = f(X)
    assert np.allclose(f(-X), -base, rtol=0, atol=1e-14)
    assert np.allclose(f(3.7 * X), base, rtol=0, atol=1e-13)
    assert np.allclose(f(X.T), base.T, rtol=0, atol=1e-13)
    Z = np.zeros((5, 9))
    assert np.array_equal(oracle.muon_orthogonalize(Z, oracle.QUINTIC, 5, eps=1e-7), Z)
    L = rng.standard_normal((12, 3)) @ rng.standard_normal((3, 40))
    s = np.linalg.svd(f(L), compute_uv=False)
    assert np.sum(s > 1e-8 * s[0]) == 3


def test_ema_and_accumulating_momentum_give_the_same_update():
    """EMA M ← βM + (1−β)g from zero state equals (1−β)·(accumulated M) at
    every step, and the Frobenius normalisation removes the factor."""
    rng = np.random.default_rng(41)
    beta = 0.95
    acc = np.zeros((6, 20))
    ema = np.zeros((6, 20))
    for _ in range(4):
        g = rng.standard_normal((6, 20))
        acc = beta * acc + g
        ema = beta * ema + (1 - beta) * g
        assert np.allclose(ema, (1 - beta) * acc, rtol=1e-13, atol=1e-15)
        u1 = oracle.muon_orthogonalize(acc, oracle.QUINTIC, 5, eps=0.0)
        u2 = oracle.muon_orthogonalize(ema, oracle.QUINTIC, 5, eps=0.0)
        assert np.allclose(u1, u2, rtol=0, atol=1e-13)


# -- momentum, rounding and the full step ---------------------------------------

def test_momentum_update_exact_small_values():
    M = np.array([[2.0, -1.0], [0.0, 4.0]], np.float32)
    g = np.array([[1.0, 1.0], [-3.0, 0.5]], np.float32)
    got = oracle.momentum_update(M, g, 0.5)
    assert got.dtype == np.float32
    assert np.array_equal(got, np.array([[2.0, 0.5], [-3.0, 2.5]], np.float32))


def test_bf16_round_matches_torch_on_fp32_values():
    rng = np.random.default_rng(51)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 lies exactly between bf16 neighbours 1 and 1 + 2^-7: even is 1.
    assert oracle.bf16_round(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3·2^-8 lies between 1 + 2^-7 and 1 + 2^-6: even mantissa is 1 + 2^-6.
    assert oracle.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert oracle.bf16_round(-(1.0 + 2.0 ** -8 + 2.0 ** -30)) == -(1.0 + 2.0 ** -7)
    assert oracle.bf16_round(0.0) == 0.0
    assert np.isinf(oracle.bf16_round(1e39))


def test_lr_shape_scale_values():
    # 18944/3584 = 37/7 and 2.2990681² = 5.2857140
    assert oracle.lr_shape_scale(18944, 3584) == pytest.approx(2.2990681, abs=1e-6)
    assert oracle.lr_shape_scale(3584, 18944) == 1.0
    assert oracle.lr_shape_scale(3584, 3584) == 1.0
    assert oracle.lr_shape_scale(512, 3584) == 1.0


@pytest.mark.parametrize("rows,cols", [(6, 20), (20, 6), (9, 9)])
def test_muon_step_rank_one_closed_form(rows, cols):
    """g = u·vᵀ, M = 0: M' = g, X₀ has one singular value 1, so
    O = φ^5(1)·û·v̂ᵀ and W' = bf16(W − lr·√max(1, rows/cols)·O)."""
    rng = np.random.default_rng(rows * 100 + cols)
    # small integers keep u·vᵀ exactly rank one after the cast to fp32
    u = rng.integers(-8, 9, rows).astype(np.float64)
    v = rng.integers(-8, 9, cols).astype(np.float64) / 64.0
    u[0], v[0] = 3.0, 0.5
    g = np.outer(u, v).astype(np.float32)
    assert np.array_equal(g.astype(np.float64), np.outer(u, v))
    W = oracle.bf16_round(rng.standard_normal((rows, cols)) * 0.02)
    M = np.zeros((rows, cols), np.float32)
    W_new, M_new, O = oracle.muon_step(W, g, M, 0.95, 0.02, oracle.QUINTIC, 5, 0.0)
    assert np.array_equal(M_new, g)
    g64 = g.astype(np.float64)
    O_want = oracle.scalar_map(1.0, oracle.QUINTIC, 5) * g64 / np.linalg.norm(g64)
    assert np.allclose(O, O_want, rtol=1e-12, atol=1e-15)
    sc = math.sqrt(max(1.0, rows / cols))
    assert np.array_equal(W_new, oracle.bf16_round(W - 0.02 * sc * O_want))


# -- the optimiser variants (Nesterov input, decoupled weight decay) ----------

def _two_rank_ones(rows, cols):
    """e₁ = (1, 1, 0, …), e₂ = (1, −1, 0, …), f₁ = (1, 0, 1, 0, …),
    f₂ = (0, 1, 0, 1, 0, …): h_i = e_i·f_iᵀ / 2 are rank-one with singular
    value 1, orthogonal row and column spaces and disjoint supports, so
    a·h₁ + b·h₂ has singular values |a|, |b|, NS acts on each independently,
    and every entry is exactly a or ±b (no rounding mixes the two)."""
    e1 = np.zeros(rows); e1[:2] = [1, 1]
    e2 = np.zeros(rows); e2[:2] = [1, -1]
    f1 = np.zeros(cols); f1[[0, 2]] = 1
    f2 = np.zeros(cols); f2[[1, 3]] = 1
    return np.outer(e1, f1) / 2, np.outer(e2, f2) / 2


@pytest.mark.parametrize("nesterov", [False, True])
def test_variants_closed_form_on_two_orthogonal_rank_ones(nesterov):
    """Two steps from M = 0 with g₁ = 4·h₁, then g₂ = 6·h₂ (exact in fp32):
    M'₂ = b₁·h₁ + 6·h₂ with b₁ = fp32(4β) (the stored state is fp32), so the
    plain input has singular values (b₁, 6) and the Nesterov input
    g₂ + β·M'₂ has (β·b₁, 6(1 + β)).  After Frobenius normalisation each
    singular value maps through φ^5, so O is known in closed form; a
    Nesterov input taken as M' (or the plain input as g + β·M') changes the
    ratio of the two singular values and fails."""
    rows, cols = 9, 14
    h1, h2 = _two_rank_ones(rows, cols)
    beta, lr, eps = 0.95, 0.02, 0.0
    g1, g2 = (4.0 * h1).astype(np.float32), (6.0 * h2).astype(np.float32)
    W = np.zeros((rows, cols))
    M = np.zeros((rows, cols), np.float32)
    _, M, _ = oracle.muon_step(W, g1, M, beta, lr, oracle.QUINTIC, 5, eps, nesterov=nesterov)
    _, M, O = oracle.muon_step(W, g2, M, beta, lr, oracle.QUINTIC, 5, eps, nesterov=nesterov)
    b1 = float(np.float32(4.0 * beta))
    assert np.array_equal(M.astype(np.float64), b1 * h1 + 6.0 * h2)

    def closed(s1, s2):
        nrm = math.hypot(s1, s2)
        return (oracle.scalar_map(s1 / nrm, oracle.QUINTIC, 5) * h1 +
                oracle.scalar_map(s2 / nrm, oracle.QUINTIC, 5) * h2)

    plain, nest = (b1, 6.0), (beta * b1, 6.0 * (1 + beta))
    want, wrong = (closed(*nest), closed(*plain)) if nesterov else (closed(*plain), closed(*nest))
    assert np.allclose(O, want, rtol=0, atol=1e-12)
    assert not np.allclose(O, wrong, rtol=0, atol=1e-3)


def test_nesterov_first_step_equals_plain():
    """From M = 0 the Nesterov input is (1 + β)·g, a positive multiple of the
    plain input, and Frobenius normalisation removes the factor."""
    rng = np.random.default_rng(5)
    g = (rng.standard_normal((12, 30)) * 1e-2).astype(np.float32)
    W = oracle.bf16_round(rng.standard_normal((12, 30)) * 0.02)
    M = np.zeros_like(g)
    a = oracle.muon_step(W, g, M, 0.9, 0.02, oracle.QUINTIC, 5, 0.0, nesterov=False)
    b = oracle.muon_step(W, g, M, 0.9, 0.02, oracle.QUINTIC, 5, 0.0, nesterov=True)
    assert np.allclose(a[2], b[2], rtol=0, atol=1e-12)
    assert np.array_equal(a[1], b[1])


def test_weight_decay_zero_gradient_halves_weights():
    """g = 0 and M = 0 give a zero update (the zero matrix normalises to 0),
    so W' = round((1 − lr·wd)·W); with lr·wd = 1/2 that is W/2, exact for
    bf16 values."""
    rng = np.random.default_rng(8)
    W = oracle.bf16_round(rng.standard_normal((7, 11)))
    z = np.zeros((7, 11), np.float32)
    W_new, M_new, O = oracle.muon_step(W, z, z, 0.95, 0.25, oracle.QUINTIC, 5, 1e-7, weight_decay=2.0)
    assert not O.any() and not M_new.any()
    assert np.array_equal(W_new, W / 2)


@pytest.mark.parametrize("rows,cols", [(6, 20), (20, 6)])
def test_weight_decay_rank_one_closed_form(rows, cols):
    """Rank-one gradient with decoupled decay: W' = bf16((1 − lr·wd)·W −
    lr·sc·φ^5(1)·g/‖g‖); lr·wd = 1/4 makes the decayed weights exact."""
    rng = np.random.default_rng(rows * 7 + cols)
    u = rng.integers(-8, 9, rows).astype(np.float64)
    v = rng.integers(-8, 9, cols).astype(np.float64) / 64.0
    u[0], v[0] = 3.0, 0.5
    g = np.outer(u, v).astype(np.float32)
    W = oracle.bf16_round(rng.standard_normal((rows, cols)) * 0.02)
    M = np.zeros((rows, cols), np.float32)
    W_new, _, O = oracle.muon_step(W, g, M, 0.95, 0.02, oracle.QUINTIC, 5, 0.0, weight_decay=12.5)
    g64 = g.astype(np.float64)
    O_want = oracle.scalar_map(1.0, oracle.QUINTIC, 5) * g64 / np.linalg.norm(g64)
    sc = math.sqrt(max(1.0, rows / cols))
    assert np.array_equal(W_new, oracle.bf16_round(0.75 * W - 0.02 * sc * O_want))


def test_gram_flops_by_enumeration():
    """Walk the product sequence of the Gram recursion (A², then Q-update,
    P·A, P·(P·A) as the step requires) and count 2·K flops per upper-triangle
    entry, plus the SYRK and the final dense product."""
    def count(rows, cols, steps):
        m, n = min(rows, cols), max(rows, cols)
        upper = m * (m + 1) // 2
        total = upper * 2 * n  # G = X·Xᵀ, upper triangle
        for k in range(steps):
            prods = 1  # A²
            if k >= 1:
                prods += 1  # Q ← aQ + B·Q (Q₁ = P₀ needs no product)
            if k <= steps - 2:
                prods += 2  # P·A, then P·(P·A)
            total += prods * upper * 2 * m
        total += 2 * m * m * n  # O = Q·X₀
        return total
    for rows, cols, s in [(256, 1024, 5), (1024, 256, 5), (3584, 18944, 5), (7, 3, 1), (8, 8, 2)]:
        assert oracle.gram_flops(rows, cols, s) == count(rows, cols, s)
    # the c5 matrix set total quoted in the design: 178.95 TF
    shapes = [(3584, 3584), (512, 3584), (512, 3584), (3584, 3584), (18944, 3584), (18944, 3584), (3584, 18944)]
    tot = 28 * sum(oracle.gram_flops(r, c, 5) for r, c in shapes)
    assert tot / 1e12 == pytest.approx(178.95, abs=0.01)
